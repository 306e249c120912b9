"""pkv_copy_blocks (copy-on-write block copy) and a beam-search loop on the GPU, through the
C ABI, against the oracle.

* the copy is bit-exact over both whole caches against the oracle's copy, for f32/f16/bf16,
  hd 64/128 and kv-head counts whose block size is below, equal to and a multiple of one
  work-group's range (the partial-range path and the full-range path), with repeated sources
  and padding / out-of-pool pairs (skipped);
* beam search: beams forked at arbitrary lengths and re-selected every step, one token
  appended per beam per step. The engine's allocator and the oracle's allocator run in
  lockstep (the uploaded tables and lengths and the number of copy-on-write pairs equal every
  step); on the device each step is
  one engine call (pkv_engine_beam_step: fork, free, append, the staging and the step's
  copy-on-write copies in one launch, the fused decode step, also with a shared-prefix plan,
  its shared and stream passes in the automatic form, in one launch or in two); on the host
  the oracle's copy, write and attention. Every step's output matches within the tolerance
  and both caches are bit-exact at the end.
"""

import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import allocator as OAL
from oracle import attention as OA
from oracle import cache_write as CW
from tests import gpu_helpers as G
from tests import helpers as H

pytestmark = pytest.mark.gpu


def pkv():
    import paged_kv_cache_459_amd as m
    return m


def storage(t, dtype):
    return W.to_storage_numpy(t, dtype).reshape(-1).view(np.uint8)


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


@pytest.mark.parametrize("dtype,hd,hkv", [
    ("f32", 64, 1), ("f32", 128, 3), ("f16", 128, 4), ("bf16", 64, 1), ("bf16", 128, 32),
    ("bf16", 128, 8), ("f16", 64, 5)])
def test_copy_blocks_matches_oracle(dtype, hd, hkv):
    m = pkv()
    rng = np.random.default_rng(61 + hd + hkv)
    nb = 40
    print(f"[copy] {dtype} hd{hd} hkv{hkv} nb{nb}", flush=True)
    size = nb * hkv * hd * 16
    kc = W.normal_values(rng, (size,), dtype)
    vc = W.normal_values(rng, (size,), dtype)
    perm = rng.permutation(nb)
    src = [int(b) for b in perm[:6]] + [int(perm[0]), int(perm[1]), -1, int(perm[2]), nb + 3]
    dst = [int(b) for b in perm[6:12]] + [int(perm[12]), int(perm[13]), int(perm[14]), -1,
                                            int(perm[15])]
    want_k, want_v = CW.copy_blocks(kc, vc, list(zip(src, dst)), hkv=hkv, hd=hd, bs=16,
                                    dtype=dtype)
    ks, vs = m.cache_shapes(nb, hkv, hd, G.TORCH[dtype])
    k_d = G.to_dev(kc, dtype).view(ks)
    v_d = G.to_dev(vc, dtype).view(vs)
    m.pkv_copy_blocks(k_d, v_d, dev_i32(src), dev_i32(dst), num_kv_heads=hkv, head_dim=hd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(storage(k_d, dtype), want_k.view(np.uint8))
    np.testing.assert_array_equal(storage(v_d, dtype), want_v.view(np.uint8))
    # no pairs: nothing changes
    m.pkv_copy_blocks(k_d, v_d, dev_i32([]), dev_i32([]), num_kv_heads=hkv, head_dim=hd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(storage(k_d, dtype), want_k.view(np.uint8))


def test_copy_many_pairs():
    """Thousands of pairs in one launch (grid.x = pairs)."""
    m = pkv()
    dtype, hd, hkv, nb = "bf16", 128, 8, 6000
    print(f"[copy] many pairs nb{nb}", flush=True)
    ks, vs = m.cache_shapes(nb, hkv, hd, torch.bfloat16)
    k_d = W.device_normal(ks, dtype, 71)
    v_d = W.device_normal(vs, dtype, 72)
    kc = W.to_storage_numpy(k_d, dtype).reshape(-1)
    vc = W.to_storage_numpy(v_d, dtype).reshape(-1)
    perm = np.random.default_rng(73).permutation(nb)
    pairs = list(zip(perm[:2900].tolist(), perm[3000:5900].tolist()))
    want_k, want_v = CW.copy_blocks(kc, vc, pairs, hkv=hkv, hd=hd, bs=16, dtype=dtype)
    m.pkv_copy_blocks(k_d, v_d, dev_i32(perm[:2900]), dev_i32(perm[3000:5900]),
                      num_kv_heads=hkv, head_dim=hd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(storage(k_d, dtype), want_k.view(np.uint8))
    np.testing.assert_array_equal(storage(v_d, dtype), want_v.view(np.uint8))


@pytest.mark.parametrize("dtype,hq,hkv,hd,kernel,plan,form", [
    ("bf16", 8, 2, 128, 0, False, "auto"), ("f32", 4, 4, 64, 0, False, "auto"),
    ("f16", 4, 4, 128, 0, False, "auto"), ("bf16", 8, 2, 64, 1, False, "auto"),
    ("bf16", 8, 2, 128, 0, True, "auto"), ("f16", 4, 4, 64, 0, True, "auto"),
    ("bf16", 8, 8, 128, 0, True, "one"), ("bf16", 8, 8, 128, 0, True, "two"),
    ("f16", 8, 2, 128, 1, True, "one")])
def test_beam_search_loop(dtype, hq, hkv, hd, kernel, plan, form):
    m = pkv()
    print(f"[beam] {dtype} {hq}/{hkv} hd{hd} kernel={kernel} plan={plan} form={form}",
          flush=True)
    groups, beams, steps, nb = 4, 4, 36, 160
    prompt_lens = (21, 16, 7, 40)
    rng = np.random.default_rng(81 + hd)
    order = rng.permutation(nb).astype(np.int32)
    ref = OAL.BlockAllocator(nb, 16, order)
    alloc = m.BlockAllocator(nb, 16, order)
    ks, vs = m.cache_shapes(nb, hkv, hd, G.TORCH[dtype])
    size = nb * hkv * hd * 16
    kc = np.full(size, H.NAN_BITS[dtype], H.STORAGE[dtype])
    vc = np.full(size, H.NAN_BITS[dtype], H.STORAGE[dtype])
    k_d = G.to_dev(kc, dtype).view(ks)
    v_d = G.to_dev(vc, dtype).view(vs)
    scale = 1.0 / math.sqrt(hd)
    next_id = 0
    live = []
    for g in range(groups):  # prompt, written with pkv_write; then the group's beams
        root = next_id
        next_id += 1
        ref.add_seq(root)
        alloc.add_seq(root)
        n = prompt_lens[g]
        want_slots, _ = ref.append([root], [n])
        slots, cows = alloc.append([root], [n])
        assert list(slots) == want_slots and len(cows) == 0
        k = W.normal_values(rng, (n, hkv, hd), dtype)
        v = W.normal_values(rng, (n, hkv, hd), dtype)
        kc, vc = CW.write_kv(k, v, kc, vc, np.int32(slots), hkv=hkv, hd=hd, bs=16, dtype=dtype)
        m.pkv_write(G.to_dev(k, dtype), G.to_dev(v, dtype), k_d, v_d, dev_i32(slots))
        row = []
        for _ in range(beams):
            ref.fork(root, next_id)
            alloc.fork(root, next_id)
            row.append(next_id)
            next_id += 1
        ref.free_seq(root)
        alloc.free(root)
        live.append(row)
    # every device step is one engine call: re-selection (fork, free), append, copy-on-write
    # copies, the fused decode step
    B = groups * beams
    prev = m.pkv_set_attn_kernel(kernel)
    eng = m.Engine(alloc, k_d, v_d, num_q_heads=hq, num_kv_heads=hkv, head_dim=hd,
                   max_batch=B, max_context_len=16 * 8, plan=plan, shared_launch=form)
    eng.adopt([s for row in live for s in row])
    dt = G.TORCH[dtype]
    q_d = torch.empty((B, hq, hd), dtype=dt, device="cuda")
    kn_d = torch.empty((B, hkv, hd), dtype=dt, device="cuda")
    vn_d = torch.empty((B, hkv, hd), dtype=dt, device="cuda")
    out = torch.empty((B, hq, hd), dtype=dt, device="cuda")
    total_cows = planned = 0
    try:
        for step in range(steps):
            parents = children = None
            if step > 0:
                pick = W.beam_parents(rng, groups, beams)
                parents = (np.arange(groups)[:, None] * beams + pick).reshape(-1)
                children = np.arange(next_id, next_id + B, dtype=np.int64)
                new_live = []
                for g in range(groups):
                    row = []
                    for p in pick[g]:
                        ref.fork(live[g][p], next_id)
                        row.append(next_id)
                        next_id += 1
                    for s in live[g]:
                        ref.free_seq(s)
                    new_live.append(row)
                live = new_live
            seqs = [s for row in live for s in row]
            want_slots, want_cows = ref.append(seqs, [1] * len(seqs))
            mb = max(len(ref.blocks[s]) for s in seqs)
            want_tables, want_lens = ref.tables(seqs, mb)
            q = W.normal_values(rng, (len(seqs), hq, hd), dtype)
            k_new = W.normal_values(rng, (len(seqs), hkv, hd), dtype)
            v_new = W.normal_values(rng, (len(seqs), hkv, hd), dtype)
            # oracle: copy, write, attend
            kc, vc = CW.copy_blocks(kc, vc, want_cows, hkv=hkv, hd=hd, bs=16, dtype=dtype)
            kc, vc = CW.write_kv(k_new, v_new, kc, vc, np.int32(want_slots), hkv=hkv, hd=hd,
                                 bs=16, dtype=dtype)
            want = OA.decode_attention(q, kc, vc, want_tables, want_lens, scale=scale, hkv=hkv,
                                       hd=hd, bs=16, dtype=dtype)
            q_d.copy_(G.to_dev(q, dtype).view(q_d.shape))
            kn_d.copy_(G.to_dev(k_new, dtype).view(kn_d.shape))
            vn_d.copy_(G.to_dev(v_new, dtype).view(vn_d.shape))
            info = eng.beam_step(q_d, kn_d, vn_d, out, scale=scale, parents=parents,
                                 children=children)
            torch.cuda.synchronize()
            assert list(eng.running()) == seqs
            assert int(info[0]) == B and int(info[5]) == len(want_cows)
            planned += int(info[4]) > 0
            last = eng.last()
            tables = np.where(last["tables"] >= 0, last["tables"] & ~0x40000000, -1)
            np.testing.assert_array_equal(tables[:, :mb], np.int32(want_tables))
            assert np.all(tables[:, mb:] == -1)
            np.testing.assert_array_equal(last["lens"], np.int32(want_lens))
            total_cows += len(want_cows)
            G.assert_close(G.gpu_f64(out, dtype), want, dtype, f"beam step {step}")
        eng.sync()
    finally:
        eng.close()
        m.pkv_set_attn_kernel(prev)
    assert total_cows > 0
    assert planned > 0 or not plan
    np.testing.assert_array_equal(storage(k_d, dtype), kc.view(np.uint8))
    np.testing.assert_array_equal(storage(v_d, dtype), vc.view(np.uint8))
    assert alloc.num_free() == ref.num_free()
