"""Decode with a shared-prefix plan (pkv_decode_plan + pkv_decode_planned) on the GPU, through
the C ABI, against the oracle.

Batches are shaped like the pages' sharing cases: a common prefix with private tails, beam
groups (a prefix shared by all, tails shared within a group, each beam's own last block), and
a mixed batch (a shared block that is only partly filled, sequences whose every block is
shared, unrelated rows, an empty row). Each physical block's content is drawn once, so
sharers see the same K/V; slots no sharer reaches hold NaN.

* plain and fused (newest token appended) decode match the oracle within the tolerance, for
  both stream kernels, MHA and GQA (G = 1..16), hd 64/128, f16/bf16, and any worker count;
* the fused step's caches are bit-exact against the oracle's write;
* the whole step, the passes apart and the shared and stream passes in one launch give the
  same bits (output and, appending, caches);
* a float32 plan (no runs) gives exactly the unplanned result;
* the full-size prefix-shared and beam batches, sampled rows against the oracle.
"""

import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from oracle import cache_write as CW
from oracle import layout as OL
from tests import gpu_helpers as G
from tests import helpers as H
from tests.test_plan import case

pytestmark = pytest.mark.gpu


def pkv():
    import paged_kv_cache_459_amd as m
    return m


def fill_shared(rng, tables, lens, nb, hq, hkv, hd, dtype):
    """Caches where every used physical block's tokens are drawn once (NaN elsewhere)."""
    size = nb * hkv * hd * 16
    kc = np.full(size, H.NAN_BITS[dtype], H.STORAGE[dtype])
    vc = np.full(size, H.NAN_BITS[dtype], H.STORAGE[dtype])
    kv, vv = OL.token_slot_views(kc, vc, hkv, hd, 16, dtype)
    reach = {}
    for row, n in zip(tables, lens):
        for j in range(-(-int(n) // 16)):
            e = int(row[j])
            b = e & ~0x40000000
            if e >= 0 and b < nb:
                reach[b] = max(reach.get(b, 0), min(16, int(n) - 16 * j))
    for b in sorted(reach):
        t = reach[b]
        kv[b, :t] = W.normal_values(rng, (t,) + kv.shape[2:], dtype)
        vv[b, :t] = W.normal_values(rng, (t, hkv, hd), dtype)
    q = W.normal_values(rng, (len(lens), hq, hd), dtype)
    return q, kc, vc


def run_planned(m, q, kc, vc, tables, lens, nb, hq, hkv, hd, dtype, scale, *, W=None,
                k_new=None, v_new=None, passes=(0,)):
    dt = G.TORCH[dtype]
    ks, vs = m.cache_shapes(nb, hkv, hd, dt)
    kd = G.to_dev(kc, dtype).view(ks)
    vd = G.to_dev(vc, dtype).view(vs)
    qd = G.to_dev(q, dtype)
    td = torch.from_numpy(np.ascontiguousarray(tables, np.int32)).cuda()
    ld = torch.from_numpy(np.ascontiguousarray(lens, np.int32)).cuda()
    max_ctx = 16 * tables.shape[1]
    plan = m.pkv_decode_plan(tables, lens, num_q_heads=hq, num_kv_heads=hkv, num_blocks=nb,
                             max_context_len=max_ctx, dtype=dt, max_group=16)
    plan_dev = torch.from_numpy(plan.copy()).cuda()
    W = W or m.pkv_decode_num_workers(hq, hkv, hd, dt)
    nbytes = m.pkv_decode_planned_workspace_bytes(len(lens), hq, hkv, hd, dt, W, plan)
    assert nbytes > 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(qd)
    kn = None if k_new is None else G.to_dev(k_new, dtype)
    vn = None if v_new is None else G.to_dev(v_new, dtype)
    for ps in passes:
        m.pkv_decode_planned(qd, kd, vd, td, ld, plan, plan_dev, num_kv_heads=hkv, scale=scale,
                             max_context_len=max_ctx, num_workers=W, workspace=ws, k_new=kn,
                             v_new=vn, out=out, passes=ps)
    torch.cuda.synchronize()
    return out, kd, vd, plan


SHAPES = [("f16", 8, 8, 128, 0), ("bf16", 8, 8, 64, 0), ("bf16", 28, 4, 128, 0),
          ("f16", 16, 8, 128, 0), ("bf16", 32, 2, 128, 0), ("bf16", 8, 4, 128, 1),
          ("f16", 32, 32, 128, 2), ("bf16", 4, 4, 64, 2)]


@pytest.mark.parametrize("kind", ["prefix", "beam", "mixed", "wide"])
@pytest.mark.parametrize("dtype,hq,hkv,hd,kernel", SHAPES)
def test_planned_matches_oracle(kind, dtype, hq, hkv, hd, kernel):
    m = pkv()
    print(f"[planned] {kind} {dtype} {hq}/{hkv} hd{hd} kernel={kernel}", flush=True)
    rng = np.random.default_rng(900 + hq + hd)
    tables, lens, nb = case(rng, kind)
    q, kc, vc = fill_shared(rng, tables, lens, nb, hq, hkv, hd, dtype)
    scale = 1.0 / math.sqrt(hd)
    prev = m.pkv_set_attn_kernel(kernel)
    try:
        out, _, _, plan = run_planned(m, q, kc, vc, tables, lens, nb, hq, hkv, hd, dtype, scale)
    finally:
        m.pkv_set_attn_kernel(prev)
    if hq // hkv <= 16:
        assert plan[4] > 0  # the batch has runs: the shared pass ran
    # rows whose blocks are all in the pool (an entry outside it leaves the row undefined)
    rows = [s for s, n in enumerate(lens)
            if all(0 <= (int(e) & ~0x40000000) < nb and int(e) >= 0
                   for e in tables[s, :-(-int(n) // 16)])]
    want = OA.decode_attention(q[rows], kc, vc, tables[rows] & ~0x40000000, lens[rows],
                               scale=scale, hkv=hkv, hd=hd, bs=16, dtype=dtype)
    got = G.gpu_f64(out, dtype)[rows]
    G.assert_close(got, want, dtype, f"planned {kind}")


@pytest.mark.parametrize("W", [4, 12, 64, 1024])
@pytest.mark.parametrize("kind", ["prefix", "beam"])
@pytest.mark.parametrize("dtype,hq,hkv,hd,kernel", [("bf16", 8, 8, 128, 0),
                                                    ("bf16", 28, 4, 128, 0)])
def test_planned_append_any_worker_count(W, kind, dtype, hq, hkv, hd, kernel):
    """Fused newest-token step with a plan: output within tolerance of the oracle (write,
    then attend), caches bit-exact, for cut and whole private segments."""
    m = pkv()
    print(f"[planned append] W={W} {kind} {dtype} {hq}/{hkv}", flush=True)
    rng = np.random.default_rng(950 + W)
    tables, lens, nb = case(rng, kind)
    q, kc, vc = fill_shared(rng, tables, lens, nb, hq, hkv, hd, dtype)
    B = len(lens)
    k_new = W_.normal_values(rng, (B, hkv, hd), dtype)
    v_new = W_.normal_values(rng, (B, hkv, hd), dtype)
    slots = np.array([int(tables[s, (int(n) - 1) // 16]) * 16 + (int(n) - 1) % 16
                      for s, n in enumerate(lens)], np.int32)
    prev = m.pkv_set_attn_kernel(kernel)
    try:
        out, kd, vd, _ = run_planned(m, q, kc, vc, tables, lens, nb, hq, hkv, hd, dtype, 0.08,
                                     W=W, k_new=k_new, v_new=v_new)
    finally:
        m.pkv_set_attn_kernel(prev)
    kc2, vc2 = CW.write_kv(k_new, v_new, kc, vc, slots, hkv=hkv, hd=hd, bs=16, dtype=dtype)
    want = OA.decode_attention(q, kc2, vc2, tables, lens, scale=0.08, hkv=hkv, hd=hd, bs=16,
                               dtype=dtype)
    G.assert_close(G.gpu_f64(out, dtype), want, dtype, f"planned append W={W}")
    np.testing.assert_array_equal(W_.to_storage_numpy(kd, dtype).reshape(-1).view(np.uint8),
                                  kc2.view(np.uint8))
    np.testing.assert_array_equal(W_.to_storage_numpy(vd, dtype).reshape(-1).view(np.uint8),
                                  vc2.view(np.uint8))


W_ = W  # the workloads module (the parameter above shadows the name W)


# append mode needs each newest token in a private block (the mixed batch shares whole rows)
@pytest.mark.parametrize("kind,append", [("beam", False), ("mixed", False), ("beam", True),
                                         ("prefix", True)])
@pytest.mark.parametrize("dtype,hq,hkv,hd,kernel", [
    ("bf16", 8, 8, 128, 0), ("f16", 28, 4, 128, 0), ("f16", 8, 4, 128, 1), ("f16", 4, 4, 64, 0),
    ("bf16", 8, 2, 64, 1)])
def test_pass_forms_give_the_same_bits(kind, append, dtype, hq, hkv, hd, kernel):
    """The whole step (pass 0), the passes apart (1, 2, 3) and the shared and stream passes in
    one launch (5, 3; two launches where the vector stream kernel does not run): the same
    output bits, and in append mode the same caches."""
    m = pkv()
    print(f"[planned forms] append={append} {kind} {dtype} {hq}/{hkv} hd{hd} kernel={kernel}",
          flush=True)
    rng = np.random.default_rng(970)
    tables, lens, nb = case(rng, kind)
    q, kc, vc = fill_shared(rng, tables, lens, nb, hq, hkv, hd, dtype)
    B = len(lens)
    kn = vn = None
    if append:
        kn = W_.normal_values(rng, (B, hkv, hd), dtype)
        vn = W_.normal_values(rng, (B, hkv, hd), dtype)
    prev = m.pkv_set_attn_kernel(kernel)
    try:
        runs = [run_planned(m, q, kc, vc, tables, lens, nb, hq, hkv, hd, dtype, 0.1,
                            k_new=kn, v_new=vn, passes=ps)
                for ps in ((0,), (1, 2, 3), (5, 3), (4, 3))]
    finally:
        m.pkv_set_attn_kernel(prev)
    ref = runs[1]
    for got in runs[:1] + runs[2:]:
        for a, b in zip(got[:3], ref[:3]):  # out, k cache, v cache
            np.testing.assert_array_equal(W_.to_storage_numpy(a, dtype).view(np.uint8),
                                          W_.to_storage_numpy(b, dtype).view(np.uint8))


def test_float32_plan_equals_unplanned_bits():
    m = pkv()
    rng = np.random.default_rng(980)
    tables, lens, nb = case(rng, "prefix")
    q, kc, vc = fill_shared(rng, tables, lens, nb, 4, 2, 64, "f32")
    out, kd, vd, plan = run_planned(m, q, kc, vc, tables, lens, nb, 4, 2, 64, "f32", 0.1)
    assert plan[4] == 0
    ref = m.pkv_decode_attn(G.to_dev(q, "f32"), kd, vd,
                            torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(),
                            num_kv_heads=2, scale=0.1, max_context_len=16 * tables.shape[1])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32),
                                  ref.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("beams", [False, True])
def test_full_size_prefix_shared(beams):
    """The prefix-shared batch at its real shape (128 sequences, 2000-token prefix, MHA 32 x
    128, bf16), and its 4-way beam variant, planned; sampled rows against the oracle."""
    m = pkv()
    print(f"[planned full size] beams={beams}", flush=True)
    rng = np.random.default_rng(990)
    B, hq, hd, pre = 128, 32, 128, 125
    if beams:
        tails = rng.integers(16, 512, size=B // 4, endpoint=True)
        lens = np.repeat(2000 + tails, 4).astype(np.int32) + 1
    else:
        lens = (2000 + rng.integers(16, 512, size=B, endpoint=True)).astype(np.int32)
    mb = -(-int(lens.max()) // 16)
    nb = 40000
    free = iter(rng.permutation(np.arange(pre, nb)))
    tables = np.full((B, mb), -1, np.int32)
    for s in range(B):
        tables[s, :pre] = np.arange(pre)
    if beams:
        for g in range(B // 4):
            n = int(lens[4 * g])
            tail = [next(free) for _ in range(-(-n // 16) - 1 - pre)]
            for b in range(4):
                s = 4 * g + b
                tables[s, pre:pre + len(tail)] = tail
                tables[s, pre + len(tail)] = next(free)
    else:
        for s in range(B):
            for j in range(pre, -(-int(lens[s]) // 16)):
                tables[s, j] = next(free)
    dt = torch.bfloat16
    ks, vs = m.cache_shapes(nb, hq, hd, dt)
    kd = W_.device_normal(ks, "bf16", 991)
    vd = W_.device_normal(vs, "bf16", 992)
    qd = W_.device_normal((B, hq, hd), "bf16", 993)
    td = torch.from_numpy(tables).cuda()
    ld = torch.from_numpy(lens).cuda()
    plan = m.pkv_decode_plan(tables, lens, num_q_heads=hq, num_kv_heads=hq, num_blocks=nb,
                             max_context_len=16 * mb, dtype=dt)
    assert plan[4] > 0
    plan_dev = torch.from_numpy(plan.copy()).cuda()
    Wk = m.pkv_decode_num_workers(hq, hq, hd, dt)
    ws = torch.empty(m.pkv_decode_planned_workspace_bytes(B, hq, hq, hd, dt, Wk, plan),
                     dtype=torch.uint8, device="cuda")
    out = m.pkv_decode_planned(qd, kd, vd, td, ld, plan, plan_dev, num_kv_heads=hq, scale=0.088,
                               max_context_len=16 * mb, num_workers=Wk, workspace=ws)
    torch.cuda.synchronize()
    for s in [0, 1, 5, 64, 127] + list(rng.choice(B, size=3, replace=False)):
        n = int(lens[s])
        c = -(-n // 16)
        ids = torch.from_numpy(tables[s, :c].astype(np.int64)).cuda()
        kh = W_.to_storage_numpy(kd.index_select(0, ids), "bf16").reshape(-1)
        vh = W_.to_storage_numpy(vd.index_select(0, ids), "bf16").reshape(-1)
        qh = W_.to_storage_numpy(qd[s:s + 1], "bf16")
        want = OA.decode_attention(qh, kh, vh, np.arange(c, dtype=np.int32)[None],
                                   np.int32([n]), scale=0.088, hkv=hq, hd=hd, bs=16, dtype="bf16")
        G.assert_close(G.gpu_f64(out[s:s + 1], "bf16"), want, "bf16", f"row {s}")


def random_tree_batch(rng, append, nb=3000):
    """A batch whose tables form a random prefix tree: a run of blocks shared by a group, the
    group split into up to four subgroups that each share a further run, and so on three
    levels deep, then private tails. Lengths end anywhere in the last block (appending: every
    sequence ends in a private block of its own)."""
    B = int(rng.integers(2, 40))
    rows = [[] for _ in range(B)]
    free = iter(rng.permutation(nb).tolist())

    def grow(members, depth):
        shared = [next(free) for _ in range(int(rng.integers(0, 20)))]
        for s in members:
            rows[s] += shared
        if depth < 3 and len(members) >= 2 and rng.random() < 0.7:
            k = int(rng.integers(1, min(4, len(members)) + 1))
            for part in np.array_split(rng.permutation(members), k):
                if len(part):
                    grow([int(x) for x in part], depth + 1)
        else:
            for s in members:
                tail = int(rng.integers(1 if append else 0, 6))
                rows[s] += [next(free) for _ in range(tail)]

    grow(list(range(B)), 0)
    mb = max(1, max(len(r) for r in rows))
    tables = np.full((B, mb), -1, np.int32)
    lens = np.zeros(B, np.int32)
    for s, r in enumerate(rows):
        tables[s, :len(r)] = r
        lens[s] = 16 * (len(r) - 1) + int(rng.integers(1, 17)) if r else 0
    return tables, lens, nb


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("dtype,hq,hkv,hd,kernel", [
    ("bf16", 8, 8, 128, 0), ("f16", 16, 16, 64, 0), ("bf16", 4, 2, 128, 0),
    ("f16", 8, 2, 128, 1), ("bf16", 32, 32, 128, 0)])
def test_random_prefix_trees(seed, dtype, hq, hkv, hd, kernel):
    """Random prefix trees, plain and appending, at several worker counts: the planned step
    matches the oracle (the write too, appending), and its pass forms give the same bits."""
    m = pkv()
    rng = np.random.default_rng(5000 + seed)
    append = seed % 2 == 1
    tables, lens, nb = random_tree_batch(rng, append)
    W = [None, 64, 36, 1024, None, 1024][seed]
    print(f"[planned tree] seed={seed} B={len(lens)} append={append} W={W} {dtype} "
          f"{hq}/{hkv} hd{hd} kernel={kernel}", flush=True)
    q, kc, vc = fill_shared(rng, tables, lens, nb, hq, hkv, hd, dtype)
    B = len(lens)
    kn = vn = None
    if append:
        kn = W_.normal_values(rng, (B, hkv, hd), dtype)
        vn = W_.normal_values(rng, (B, hkv, hd), dtype)
    prev = m.pkv_set_attn_kernel(kernel)
    try:
        runs = [run_planned(m, q, kc, vc, tables, lens, nb, hq, hkv, hd, dtype, 0.09, W=W,
                            k_new=kn, v_new=vn, passes=ps)
                for ps in ((0,), (1, 2, 3), (5, 3))]
    finally:
        m.pkv_set_attn_kernel(prev)
    for got in runs[1:]:
        for a, b in zip(got[:3], runs[0][:3]):
            np.testing.assert_array_equal(W_.to_storage_numpy(a, dtype).view(np.uint8),
                                          W_.to_storage_numpy(b, dtype).view(np.uint8))
    out, kd, vd, _ = runs[0]
    if append:
        slots = np.array([int(tables[s, (int(n) - 1) // 16]) * 16 + (int(n) - 1) % 16
                          for s, n in enumerate(lens)], np.int32)
        kc, vc = CW.write_kv(kn, vn, kc, vc, slots, hkv=hkv, hd=hd, bs=16, dtype=dtype)
        np.testing.assert_array_equal(W_.to_storage_numpy(kd, dtype).reshape(-1).view(np.uint8),
                                      kc.view(np.uint8))
        np.testing.assert_array_equal(W_.to_storage_numpy(vd, dtype).reshape(-1).view(np.uint8),
                                      vc.view(np.uint8))
    want = OA.decode_attention(q, kc, vc, tables, lens, scale=0.09, hkv=hkv, hd=hd, bs=16,
                               dtype=dtype)
    G.assert_close(G.gpu_f64(out, dtype), want, dtype, f"tree seed {seed}")
