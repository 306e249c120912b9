"""Full-size parity on the path the benchmark times, every row.

Each benchmark workload at its real shape runs one decode step exactly as bench.py launches
it: each sequence's newest K/V (k_new, v_new) is substituted by the stream pass and stored by
the merge pass (pkv_decode_append_stream + pkv_decode_append_merge at the device's default
worker count), or, for the shared-prefix batches, the planned step (pkv_decode_planned with
k_new, v_new); the beam-search batch also as the step engine runs it (pkv_engine_beam_step:
re-selection, append with copy-on-write copies, the planned step). Then:

* every output row and head is compared with the oracle (its cache write, then dense
  attention over each sequence's gathered K/V), within the tolerance;
* both caches after the step are compared bit for bit, over the whole pool, with the oracle's
  write of the newest tokens into the caches as they were before the step.

The oracle runs on the host over exact copies of the pool; sequences are split over a thread
pool (the gathers and products release the interpreter lock for most of their time).
"""

import concurrent.futures
import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import allocator as OAL
from oracle import attention as OA
from oracle import cache_write as CW
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu


def pkv():
    import paged_kv_cache_459_amd as m
    return m


def newest_slots(tables, lens):
    return np.array([int(row[(int(n) - 1) // 16]) * 16 + (int(n) - 1) % 16
                     for row, n in zip(tables, lens)], np.int32)


def oracle_all_rows(q, kc, vc, tables, lens, *, scale, hkv, hd, dtype):
    """decode_attention over every row, rows split into chunks over a thread pool."""
    B = len(lens)
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    chunks = [list(range(a, min(B, a + 4))) for a in range(0, B, 4)]

    def run(rows):
        return rows, OA.decode_attention_rows(q, kc, vc, tables, lens, rows, scale=scale,
                                              hkv=hkv, hd=hd, bs=16, dtype=dtype)
    out = np.zeros((B, q.shape[1], hd), np.float64)
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        for rows, res in ex.map(run, chunks):
            out[rows] = res
    return out


def shared_problem(name, seed):
    """The prefix-shared batch (or its 4-beam variant): lengths after the step, tables with a
    125-block common prefix, device-filled pool."""
    shape = W.SHAPES[name]
    rng = W.rng_for(seed)
    lens = W.draw_lengths(shape, rng)
    need = sum(W.blocks_for(n) for n in lens)
    nb = W.pool_blocks([16 * need])
    order = rng.permutation(nb).astype(np.int32)
    if name == "beam_search":
        tables, lens = W.beam_tables(lens[::W.BEAMS] - W.PREFIX_TOKENS, order, beams=W.BEAMS)
    else:
        tables = W.prefix_shared_tables(lens, order)
    return shape, lens.astype(np.int32), tables, nb


def step_and_check(m, shape, lens, tables, nb, seed, *, planned):
    dt = G.TORCH[shape.dtype]
    B, hq, hkv, hd = len(lens), shape.Hq, shape.Hkv, shape.hd
    mb = tables.shape[1]
    max_ctx = int(lens.max())
    k_cache, v_cache = m.alloc_caches(nb, hkv, hd, dt)
    k_cache.view(-1).copy_(W.device_normal((k_cache.numel(),), shape.dtype, seed + 1))
    v_cache.view(-1).copy_(W.device_normal((v_cache.numel(),), shape.dtype, seed + 2))
    q = W.device_normal((B, hq, hd), shape.dtype, seed + 3)
    k_new = W.device_normal((B, hkv, hd), shape.dtype, seed + 4)
    v_new = W.device_normal((B, hkv, hd), shape.dtype, seed + 5)
    kc_before = W.to_storage_numpy(k_cache, shape.dtype).reshape(-1)
    vc_before = W.to_storage_numpy(v_cache, shape.dtype).reshape(-1)
    scale = G.scale_for(hd)
    td = torch.from_numpy(tables).cuda()
    ld = torch.from_numpy(lens).cuda()
    Wk = m.pkv_decode_num_workers(hq, hkv, hd, dt)
    out = torch.empty_like(q)
    if planned:
        plan = m.pkv_decode_plan(tables, lens, num_q_heads=hq, num_kv_heads=hkv, num_blocks=nb,
                                 max_context_len=max_ctx, dtype=dt)
        assert plan[4] > 0, "the batch should be planned"
        ws = torch.empty(m.pkv_decode_planned_workspace_bytes(B, hq, hkv, hd, dt, Wk, plan),
                         dtype=torch.uint8, device="cuda")
        m.pkv_decode_planned(q, k_cache, v_cache, td, ld, plan, torch.from_numpy(plan.copy()).cuda(),
                             num_kv_heads=hkv, scale=scale, max_context_len=max_ctx,
                             num_workers=Wk, workspace=ws, k_new=k_new, v_new=v_new, out=out)
    else:
        ws = torch.empty(m.pkv_decode_stream_workspace_bytes(B, hq, hkv, hd, dt, Wk),
                         dtype=torch.uint8, device="cuda")
        m.pkv_decode_append_stream(q, k_new, v_new, k_cache, v_cache, td, ld, num_kv_heads=hkv,
                                   scale=scale, max_context_len=max_ctx, num_workers=Wk,
                                   workspace=ws, out=out)
        m.pkv_decode_append_merge(out, k_new, v_new, k_cache, v_cache, td, ld, ws,
                                  num_kv_heads=hkv, max_context_len=max_ctx, num_workers=Wk)
    torch.cuda.synchronize()
    got = G.gpu_f64(out, shape.dtype)
    kc_got = W.to_storage_numpy(k_cache, shape.dtype).reshape(-1)
    vc_got = W.to_storage_numpy(v_cache, shape.dtype).reshape(-1)
    del k_cache, v_cache, ws
    kn = W.to_storage_numpy(k_new, shape.dtype)
    vn = W.to_storage_numpy(v_new, shape.dtype)
    qh = W.to_storage_numpy(q, shape.dtype)
    kc, vc = CW.write_kv(kn, vn, kc_before, vc_before, newest_slots(tables, lens), hkv=hkv,
                         hd=hd, bs=16, dtype=shape.dtype)
    del kc_before, vc_before
    np.testing.assert_array_equal(kc_got.view(np.uint8), kc.view(np.uint8),
                                  err_msg="k_cache after the step")
    np.testing.assert_array_equal(vc_got.view(np.uint8), vc.view(np.uint8),
                                  err_msg="v_cache after the step")
    want = oracle_all_rows(qh, kc, vc, tables, lens, scale=scale, hkv=hkv, hd=hd,
                           dtype=shape.dtype)
    G.assert_close(got, want, shape.dtype, f"{shape.name}: all {B} rows x {hq} heads")


@pytest.mark.parametrize("name", ["llama2_7b", "qwen25_7b", "long_context"])
def test_timed_step_every_row(name):
    m = pkv()
    shape = W.SHAPES[name]
    print(f"[full size, timed path] {name}", flush=True)
    rng = W.rng_for(shape.seed)
    lens = W.draw_lengths(shape, rng)
    nb = W.pool_blocks(lens)
    order = rng.permutation(nb).astype(np.int32)
    tables = W.place_sequences(lens, order)
    step_and_check(m, shape, lens, tables, nb, 3000 + shape.seed, planned=False)


@pytest.mark.parametrize("name", ["prefix_shared", "beam_search"])
def test_planned_step_every_row(name):
    m = pkv()
    print(f"[full size, planned step] {name}", flush=True)
    shape, lens, tables, nb = shared_problem(name, W.SHAPES[name].seed)
    step_and_check(m, shape, lens, tables, nb, 4000 + shape.seed, planned=True)


def test_engine_beam_step_every_row():
    """The beam-search workload's engine step at full size (128 beams in 32 groups sharing a
    2000-token prefix, group tails U[16, 512]): the engine's allocator and the oracle's run the
    same re-selection, then every row and head is checked and both caches bit for bit."""
    m = pkv()
    print("[full size, engine beam step] beam_search", flush=True)
    shape = W.SHAPES["beam_search"]
    B, hq, hkv, hd = shape.B, shape.Hq, shape.Hkv, shape.hd
    rng = W.rng_for(shape.seed)
    lens0 = W.draw_lengths(shape, rng)
    nb = 2048
    order = rng.permutation(nb).astype(np.int32)
    ref = OAL.BlockAllocator(nb, 16, order)
    alloc = m.BlockAllocator(nb, 16, order)
    groups = B // W.BEAMS
    parent = 10_000_000
    roots = list(range(parent + 1, parent + 1 + groups))
    seqs = list(range(B))
    for a in (ref, alloc):  # prefix, group tails, beams (as the benchmark builds them)
        a.add_seq(parent)
        a.append([parent], [W.PREFIX_TOKENS])
        for r in roots:
            a.fork(parent, r)
        (a.free_seq if a is ref else a.free)(parent)
        a.append(roots, [int(n) - 1 - W.PREFIX_TOKENS for n in lens0[::W.BEAMS]])
        for g, r in enumerate(roots):
            for b in range(W.BEAMS):
                a.fork(r, seqs[g * W.BEAMS + b])
        for r in roots:
            (a.free_seq if a is ref else a.free)(r)
    dt = G.TORCH[shape.dtype]
    max_ctx = int(lens0.max()) + 16
    k_cache, v_cache = m.alloc_caches(nb, hkv, hd, dt)
    k_cache.view(-1).copy_(W.device_normal((k_cache.numel(),), shape.dtype, 5001))
    v_cache.view(-1).copy_(W.device_normal((v_cache.numel(),), shape.dtype, 5002))
    q = W.device_normal((B, hq, hd), shape.dtype, 5003)
    k_new = W.device_normal((B, hkv, hd), shape.dtype, 5004)
    v_new = W.device_normal((B, hkv, hd), shape.dtype, 5005)
    kc = W.to_storage_numpy(k_cache, shape.dtype).reshape(-1)
    vc = W.to_storage_numpy(v_cache, shape.dtype).reshape(-1)
    eng = m.Engine(alloc, k_cache, v_cache, num_q_heads=hq, num_kv_heads=hkv, head_dim=hd,
                   max_batch=B, max_context_len=max_ctx, plan=True)
    try:
        eng.adopt(seqs)
        pick = W.beam_parents(np.random.default_rng(shape.seed + 100), groups, W.BEAMS)
        parents = (np.arange(groups)[:, None] * W.BEAMS + pick).reshape(-1)
        children = np.arange(B, 2 * B, dtype=np.int64)
        out = torch.empty_like(q)
        info = eng.beam_step(q, k_new, v_new, out, scale=G.scale_for(hd), parents=parents,
                             children=children)
        torch.cuda.synchronize()
        got_lens, got_tables = eng.last_tables()
        assert int(info[4]) > 0, "the step should run a shared-prefix plan"
        # the oracle's re-selection, append, copy-on-write copies and newest-token writes
        for i in range(B):
            ref.fork(seqs[parents[i]], int(children[i]))
        for s_ in seqs:
            ref.free_seq(s_)
        kids = [int(c) for c in children]
        slots, cows = ref.append(kids, [1] * B)
        assert int(info[5]) == len(cows) > 0
        mb = got_tables.shape[1]
        tables, lens = ref.tables(kids, mb)
        tables = np.int32(tables)
        np.testing.assert_array_equal(np.where(got_tables >= 0, got_tables & ~0x40000000, -1),
                                      tables)
        np.testing.assert_array_equal(got_lens, np.int32(lens))
        kc, vc = CW.copy_blocks(kc, vc, cows, hkv=hkv, hd=hd, bs=16, dtype=shape.dtype)
        kn = W.to_storage_numpy(k_new, shape.dtype)
        vn = W.to_storage_numpy(v_new, shape.dtype)
        kc, vc = CW.write_kv(kn, vn, kc, vc, np.int32(slots), hkv=hkv, hd=hd, bs=16,
                             dtype=shape.dtype)
        np.testing.assert_array_equal(
            W.to_storage_numpy(k_cache, shape.dtype).reshape(-1).view(np.uint8),
            kc.view(np.uint8), err_msg="k_cache after the step")
        np.testing.assert_array_equal(
            W.to_storage_numpy(v_cache, shape.dtype).reshape(-1).view(np.uint8),
            vc.view(np.uint8), err_msg="v_cache after the step")
        got = G.gpu_f64(out, shape.dtype)
        want = oracle_all_rows(W.to_storage_numpy(q, shape.dtype), kc, vc, tables,
                               np.int32(lens), scale=G.scale_for(hd), hkv=hkv, hd=hd,
                               dtype=shape.dtype)
        G.assert_close(got, want, shape.dtype, f"engine beam step: all {B} rows x {hq} heads")
    finally:
        eng.close()
