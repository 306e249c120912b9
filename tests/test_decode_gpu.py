"""pkv_decode_attn (and its two passes) on the GPU against the float64 oracle.

Tolerance (max-abs over all outputs): 1e-5 for f32, 1e-2 for f16/bf16 (fp32 accumulation).
Bit-exact on the GPU: placement permutations, shared vs duplicated blocks, repeated runs,
garbage table entries past a sequence's length, one-token contexts (out == V).
Unused cache slots hold NaN in every small-problem test.
"""

import math
import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from oracle import cache_write as CW
from oracle.allocator import BlockAllocator as OracleAlloc
from tests import gpu_helpers as G
from tests import helpers as H

pytestmark = pytest.mark.gpu

RAGGED = [0, 1, 2, 15, 16, 17, 31, 100, 511, 512, 513, 1000, 1500, 2100]


def pkv():
    import paged_kv_cache_459_amd as m
    return m


def run_decode(p, d, scale, kernel=0, max_ctx=None, max_blocks=None):
    m = pkv()
    prev = m.pkv_set_attn_kernel(kernel)
    try:
        mc = max_ctx if max_ctx is not None else G.max_context(p["lengths"])
        out = m.pkv_decode_attn(d["q"], d["k_cache"], d["v_cache"], d["tables"], d["lens"],
                                num_kv_heads=p["hkv"], scale=scale, max_context_len=mc)
        torch.cuda.synchronize()
    finally:
        m.pkv_set_attn_kernel(prev)
    return out


CASES = [
    # dtype, Hq, Hkv, hd, kernel (0 auto, 1 vector, 2 matrix-core)
    ("f32", 2, 2, 64, 0),
    ("f32", 4, 2, 128, 0),
    ("f16", 4, 4, 128, 0),
    ("f16", 4, 4, 64, 0),
    ("bf16", 4, 4, 128, 0),
    ("f16", 8, 2, 128, 0),
    ("f16", 8, 2, 128, 1),
    ("bf16", 7, 1, 128, 0),
    ("bf16", 7, 1, 128, 1),
    ("bf16", 8, 2, 64, 2),
    ("bf16", 32, 2, 128, 0),
    ("f16", 34, 2, 64, 0),  # G = 17: vector kernel
    ("bf16", 4, 4, 128, 2),  # matrix-core kernel on multi-head attention
]


@pytest.mark.parametrize("dtype,hq,hkv,hd,kernel", CASES)
def test_decode_parity_ragged(dtype, hq, hkv, hd, kernel):
    print(f"[decode] {dtype} Hq={hq} Hkv={hkv} hd={hd} kernel={kernel}", flush=True)
    rng = np.random.default_rng(1000 + hq * 7 + hkv + hd)
    p = H.random_problem(rng, RAGGED, hq, hkv, hd, dtype)
    scale = 1.0 / math.sqrt(hd)
    want = G.oracle_out(p, scale)
    got = G.gpu_f64(run_decode(p, G.device_problem(p), scale, kernel), dtype)
    G.assert_close(got, want, dtype, f"{dtype} {hq}/{hkv} hd{hd} k{kernel}")


def test_tiny_config():
    """4 sequences of {1, 15, 16, 37} tokens, 2 q / 2 kv heads, hd 64, f32, a 16-block pool
    assigned by a seeded random permutation; plus the block table [5, 12, 3] for the
    37-token sequence (the pages' block-table example)."""
    shape = W.SHAPES["tiny"]
    rng = W.rng_for(shape.seed)
    lens = W.draw_lengths(shape, rng)
    p = H.random_problem(rng, lens, 2, 2, 64, "f32", nb=W.TINY_POOL)
    scale = 1 / 8
    G.assert_close(G.gpu_f64(run_decode(p, G.device_problem(p), scale), "f32"),
                   G.oracle_out(p, scale), "f32", "tiny")
    # fixed-table variant
    tables = np.full((4, 3), -1, np.int32)
    tables[0, :1] = [0]
    tables[1, :1] = [1]
    tables[2, :1] = [2]
    tables[3, :3] = [5, 12, 3]
    k, v = H.build_caches(p["seq_k"], p["seq_v"], tables, lens, 16, 2, 64, 16, "f32")
    p2 = dict(p, tables=tables, k_cache=k, v_cache=v)
    G.assert_close(G.gpu_f64(run_decode(p2, G.device_problem(p2), scale), "f32"),
                   G.oracle_out(p2, scale), "f32", "tiny fixed table")


@pytest.mark.parametrize("dtype,hq,hkv,kernel", [("f32", 2, 2, 0), ("f16", 4, 4, 0),
                                                 ("bf16", 8, 2, 0), ("bf16", 8, 2, 1),
                                                 ("f16", 8, 1, 2)])
def test_single_token_context_returns_v_bit_exact(dtype, hq, hkv, kernel):
    rng = np.random.default_rng(3)
    p = H.random_problem(rng, [1, 1, 1, 1], hq, hkv, 128, dtype)
    got = W.to_storage_numpy(run_decode(p, G.device_problem(p), 0.3, kernel), dtype)
    G_ = hq // hkv
    for i in range(4):
        want = np.repeat(p["seq_v"][i][0], G_, axis=0)
        np.testing.assert_array_equal(got[i].view(np.uint8), want.view(np.uint8))


def test_zero_length_rows_are_zero():
    rng = np.random.default_rng(4)
    p = H.random_problem(rng, [0, 20, 0, 700], 8, 2, 128, "bf16")
    got = G.gpu_f64(run_decode(p, G.device_problem(p), 0.1), "bf16")
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    G.assert_close(got, G.oracle_out(p, 0.1), "bf16", "zero rows")


@pytest.mark.parametrize("dtype,hq,hkv,kernel", [("f16", 4, 4, 0), ("bf16", 8, 2, 0),
                                                 ("bf16", 8, 2, 1), ("f32", 2, 1, 0)])
def test_placement_shared_and_repeat_are_bit_exact(dtype, hq, hkv, kernel):
    rng = np.random.default_rng(5)
    hd = 128
    lens = [37, 512, 700, 1300]
    base = H.random_problem(rng, lens, hq, hkv, hd, dtype, nb=400)
    scale = 0.09
    out0 = W.to_storage_numpy(run_decode(base, G.device_problem(base), scale, kernel), dtype)
    # repeat
    out1 = W.to_storage_numpy(run_decode(base, G.device_problem(base), scale, kernel), dtype)
    np.testing.assert_array_equal(out0.view(np.uint8), out1.view(np.uint8))
    # another placement of the same logical K/V
    order = rng.permutation(400).astype(np.int32)
    t2 = W.place_sequences(lens, order)
    k, v = H.build_caches(base["seq_k"], base["seq_v"], t2, lens, 400, hkv, hd, 16, dtype)
    p2 = dict(base, tables=t2, k_cache=k, v_cache=v)
    out2 = W.to_storage_numpy(run_decode(p2, G.device_problem(p2), scale, kernel), dtype)
    np.testing.assert_array_equal(out0.view(np.uint8), out2.view(np.uint8))
    # sequences 1..3 share the first 32 blocks (512 tokens) of sequence 1, vs private copies
    seq_k = [x.copy() for x in base["seq_k"]]
    seq_v = [x.copy() for x in base["seq_v"]]
    for i in (2, 3):
        seq_k[i][:512] = seq_k[1][:512]
        seq_v[i][:512] = seq_v[1][:512]
    shared = W.place_sequences(lens, order)
    for i in (2, 3):
        shared[i, :32] = shared[1, :32]
    dup = W.place_sequences(lens, order)
    ks, vs = H.build_caches(seq_k, seq_v, shared, lens, 400, hkv, hd, 16, dtype)
    kd, vd = H.build_caches(seq_k, seq_v, dup, lens, 400, hkv, hd, 16, dtype)
    ps = dict(base, seq_k=seq_k, seq_v=seq_v, tables=shared, k_cache=ks, v_cache=vs)
    pd = dict(base, seq_k=seq_k, seq_v=seq_v, tables=dup, k_cache=kd, v_cache=vd)
    o_s = W.to_storage_numpy(run_decode(ps, G.device_problem(ps), scale, kernel), dtype)
    o_d = W.to_storage_numpy(run_decode(pd, G.device_problem(pd), scale, kernel), dtype)
    np.testing.assert_array_equal(o_s.view(np.uint8), o_d.view(np.uint8))
    G.assert_close(H.f64(o_s, dtype), G.oracle_out(ps, scale), dtype, "shared")


def test_table_entries_past_the_length_are_ignored():
    rng = np.random.default_rng(6)
    p = H.random_problem(rng, [5, 16, 40, 600], 4, 4, 128, "f16")
    mb = 64
    t = np.full((4, mb), -1, np.int32)
    t[:, :p["tables"].shape[1]] = p["tables"]
    p = dict(p, tables=t)
    ref = W.to_storage_numpy(run_decode(p, G.device_problem(p), 0.1, max_ctx=mb * 16), "f16")
    junk = t.copy()
    for i, n in enumerate(p["lengths"]):
        junk[i, -(-int(n) // 16):] = np.array([123456789, -5, 7, 0] * mb, np.int32)[:mb - -(-int(n) // 16)]
    pj = dict(p, tables=junk)
    got = W.to_storage_numpy(run_decode(pj, G.device_problem(pj), 0.1, max_ctx=mb * 16), "f16")
    np.testing.assert_array_equal(ref.view(np.uint8), got.view(np.uint8))


def run_passes(p, d, scale, W, kernel=0, max_ctx=None, ws_fill=None):
    """Stream pass then merge pass with W workers; returns (out, workspace, kernel used)."""
    m = pkv()
    prev = m.pkv_set_attn_kernel(kernel)
    try:
        dt = G.TORCH[p["dtype"]]
        B = len(p["lengths"])
        mc = max_ctx if max_ctx is not None else G.max_context(p["lengths"])
        nbytes = m.pkv_decode_stream_workspace_bytes(B, p["hq"], p["hkv"], p["hd"], dt, W)
        ws = torch.full((nbytes,), 0xFF if ws_fill is None else ws_fill, dtype=torch.uint8,
                        device="cuda")
        out = torch.full_like(d["q"], 7.0)
        m.pkv_decode_stream(d["q"], d["k_cache"], d["v_cache"], d["tables"], d["lens"],
                            num_kv_heads=p["hkv"], scale=scale, max_context_len=mc,
                            num_workers=W, workspace=ws, out=out)
        after_stream = out.clone()
        m.pkv_decode_merge(out, ws, num_kv_heads=p["hkv"], num_workers=W)
        torch.cuda.synchronize()
        used = m.pkv_decode_kernel(p["hq"], p["hkv"], dt)
    finally:
        m.pkv_set_attn_kernel(prev)
    return out, after_stream, ws, used


@pytest.mark.parametrize("W", [4, 8, 12, 36, 64, 256, 1024, 0])
@pytest.mark.parametrize("dtype,hq,hkv,kernel", [("f32", 2, 2, 0), ("bf16", 8, 2, 0),
                                                 ("f16", 4, 4, 0), ("bf16", 8, 2, 1)])
def test_any_worker_count(W, dtype, hq, hkv, kernel):
    """Stream + merge with few workers (long ranges, several segments per wave) to many (one
    block per wave, every segment cut), against the oracle. W = 0: the device default."""
    m = pkv()
    print(f"[workers] W={W} {dtype} {hq}/{hkv} kernel={kernel}", flush=True)
    rng = np.random.default_rng(7)
    p = H.random_problem(rng, [1, 16, 47, 0, 64, 65, 300, 1025, 2000], hq, hkv, 128, dtype)
    d = G.device_problem(p)
    if W == 0:
        prev = m.pkv_set_attn_kernel(kernel)
        W = m.pkv_decode_num_workers(hq, hkv, 128, G.TORCH[dtype])
        m.pkv_set_attn_kernel(prev)
        assert W > 0 and W % 4 == 0
    out, _, _, _ = run_passes(p, d, 0.08, W, kernel)
    G.assert_close(G.gpu_f64(out, dtype), G.oracle_out(p, 0.08), dtype, f"W={W}")


@pytest.mark.parametrize("dtype,hq,hkv,kernel,W", [("f32", 2, 2, 0, 8), ("bf16", 8, 2, 0, 12),
                                                   ("bf16", 8, 2, 1, 20), ("f16", 4, 4, 0, 16),
                                                   ("f16", 7, 1, 0, 4)])
def test_stream_pieces_match_oracle(dtype, hq, hkv, kernel, W):
    """The stream pass alone: seg holds the prefix sums (exact); rows of segments inside one
    range and rows with n = 0 are final; every piece of a cut segment is (m, l, o) over its
    token range (m in base-2 units); rows of cut segments are left untouched."""
    m = pkv()
    rng = np.random.default_rng(8)
    lens = [65, 100, 0, 200, 513, 1000, 3]
    p = H.random_problem(rng, lens, hq, hkv, 128, dtype)
    d = G.device_problem(p)
    scale = 0.1
    _, after, ws, used = run_passes(p, d, scale, W, kernel)
    Hs, gs = (hkv, hq // hkv) if used == 2 else (hq, 1)
    whole, cut, seg = G.stream_cells(lens, Hs, W)
    assert cut, "this shape is meant to cut segments"
    wseg, wml, wo = (x.cpu() for x in m.split_workspace(ws, len(lens), hq, hkv, 128, W, used))
    np.testing.assert_array_equal(wseg.numpy(), seg.astype(np.int32))
    got = G.gpu_f64(after, dtype)
    want = G.oracle_out(p, scale)
    for i, n in enumerate(lens):
        if n == 0:
            assert np.all(got[i] == 0)
    for (i, s) in whole:
        heads = list(range(s * gs, (s + 1) * gs))
        G.assert_close(got[i, heads], want[i, heads], dtype, f"whole segment {(i, s)}")
    tol = G.TOL[dtype]
    for (i, s), pieces in cut.items():
        heads = list(range(s * gs, (s + 1) * gs))
        assert np.all(got[i, heads] == 7.0), "the stream pass must not write a cut row"
        for (w, slot, lo, hi) in pieces:
            om, ol, oo = OA.range_partials(p["q"], p["k_cache"], p["v_cache"], p["tables"],
                                           p["lengths"], seq=i, lo=lo, hi=hi, scale=scale,
                                           hkv=hkv, hd=128, bs=16, dtype=dtype)
            for k, h in enumerate(heads):
                gm = float(wml[w, slot, k, 0])
                gl = float(wml[w, slot, k, 1])
                go = wo[w, slot, k].double().numpy()
                wm2 = om[h] / math.log(2.0)
                assert abs(gm - wm2) <= 1e-4 * max(1.0, abs(wm2)), ((i, s), w, slot, h)
                assert abs(gl - ol[h]) <= 1e-4 * ol[h], ((i, s), w, slot, h)
                assert np.abs(go / gl - oo[h] / ol[h]).max() <= tol, ((i, s), w, slot, h)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_merge_pass_alone(dtype):
    """The merge kernel on a workspace written on the host (prefix sums of the lengths and
    random pieces for every cut segment), against the oracle's log-sum-exp recombination of
    those values; rows of uncut segments stay untouched."""
    m = pkv()
    rng = np.random.default_rng(9)
    hq, hkv, hd, W = 3, 3, 128, 8
    lens = [0, 64, 65, 300, 499, 500]
    B = len(lens)
    whole, cut, seg = G.stream_cells(lens, hq, W)
    nbytes = m.pkv_decode_stream_workspace_bytes(B, hq, hkv, hd, G.TORCH[dtype], W)
    host = torch.zeros(nbytes, dtype=torch.uint8)
    wseg, wml, wo = m.split_workspace(host, B, hq, hkv, hd, W, 1)
    wseg.copy_(torch.from_numpy(seg.astype(np.int32)))
    wml[..., 0] = torch.from_numpy(rng.normal(0, 3, (W, 2, 1)).astype(np.float32))
    wml[..., 1] = torch.from_numpy(rng.uniform(0.5, 60, (W, 2, 1)).astype(np.float32))
    wo.copy_(torch.from_numpy((rng.normal(0, 1, (W, 2, 1, hd)) *
                               wml[..., 1:].numpy()).astype(np.float32)))
    first = next(iter(cut.values()))[0]
    wml[first[0], first[1], 0, 0] = -float("inf")  # a piece with no valid token
    wml[first[0], first[1], 0, 1] = 0.0
    wo[first[0], first[1], 0] = 0.0
    out = torch.full((B, hq, hd), 7.0, dtype=G.TORCH[dtype], device="cuda")
    m.pkv_decode_merge(out, host.cuda(), num_kv_heads=hkv, num_workers=W)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    for i in range(B):
        for h in range(hq):
            if (i, h) not in cut:
                assert np.all(got[i, h] == 7.0)  # finished by the stream pass, or n = 0
                continue
            cells = [(w, slot) for (w, slot, _, _) in cut[(i, h)]]
            M2 = np.array([float(wml[w, sl, 0, 0]) for w, sl in cells])
            Lv = np.array([float(wml[w, sl, 0, 1]) for w, sl in cells])
            Ov = np.stack([wo[w, sl, 0].double().numpy() for w, sl in cells])
            want = OA.merge_partials(M2 * math.log(2.0), Lv, Ov)
            assert np.abs(got[i, h] - want).max() <= G.TOL[dtype] * max(1, np.abs(want).max())


def test_decode_step_with_allocator_and_write():
    """One decode step: allocate on demand (some sequences open a fresh block, one forks a
    shared partly-filled block and copies on write), write the new token, attend. The
    expected value uses only the oracle allocator, the oracle write and the oracle attention;
    the library's allocator must hand out the same slots, tables and copy pairs."""
    m = pkv()
    rng = np.random.default_rng(10)
    hq, hkv, hd, dtype = 8, 2, 128, "bf16"
    prefill = [15, 16, 100, 33, 47]
    nb = 40
    order = rng.permutation(nb).astype(np.int32)
    ora = OracleAlloc(nb, 16, order)
    nat = m.BlockAllocator(nb, 16, order)
    for s, n in enumerate(prefill):
        ora.add_seq(s)
        nat.add_seq(s)
        so, _ = ora.append([s], [n])
        sn, _ = nat.append([s], [n])
        assert sn.tolist() == so
    ora.fork(3, 5)  # 33 tokens: the last block holds one token and is now shared
    nat.fork(3, 5)
    seqs = [0, 1, 2, 3, 4, 5]
    so, cow_o = ora.append(seqs, [1] * 6)
    sn, cow_n = nat.append(seqs, [1] * 6)
    assert sn.tolist() == so and [tuple(c) for c in cow_n.tolist()] == cow_o and cow_o
    mb = 8
    t_o, l_o = ora.tables(seqs, mb)
    t_n, l_n = nat.tables(seqs, mb)
    assert t_n.tolist() == t_o and l_n.tolist() == l_o
    t_o = np.array(t_o, np.int32)
    # pool contents before the step: seeded values; unused slots NaN
    size = nb * hkv * hd * 16
    kc = W.normal_values(rng, (size,), dtype)
    vc = W.normal_values(rng, (size,), dtype)
    k_new = W.normal_values(rng, (6, hkv, hd), dtype)
    v_new = W.normal_values(rng, (6, hkv, hd), dtype)
    q = W.normal_values(rng, (6, hq, hd), dtype)
    # expected: copy-on-write, then the write, then attention (all oracle)
    from oracle import layout as OL
    kc_e, vc_e = kc.copy(), vc.copy()
    kv_, vv_ = OL.token_slot_views(kc_e, vc_e, hkv, hd, 16, dtype)
    for src, dst in cow_o:
        kv_[dst] = kv_[src]
        vv_[dst] = vv_[src]
    kc_e, vc_e = CW.write_kv(k_new, v_new, kc_e, vc_e, np.int32(so), hkv=hkv, hd=hd, bs=16,
                             dtype=dtype)
    want = OA.decode_attention(q, kc_e, vc_e, t_o, l_o, scale=0.1, hkv=hkv, hd=hd, bs=16,
                               dtype=dtype)
    # GPU: copy-on-write copies (torch copy of tiles), library write, library attention
    ks, vs = m.cache_shapes(nb, hkv, hd, torch.bfloat16)
    dk = G.to_dev(kc, dtype).view(ks)
    dv = G.to_dev(vc, dtype).view(vs)
    for src, dst in cow_n.tolist():
        dk[dst].copy_(dk[src])
        dv[dst].copy_(dv[src])
    m.pkv_write(G.to_dev(k_new, dtype), G.to_dev(v_new, dtype), dk, dv,
                torch.from_numpy(sn).cuda())
    out = m.pkv_decode_attn(G.to_dev(q, dtype), dk, dv, torch.from_numpy(t_n).cuda(),
                            torch.from_numpy(l_n).cuda(), num_kv_heads=hkv, scale=0.1,
                            max_context_len=mb * 16)
    torch.cuda.synchronize()
    G.assert_close(G.gpu_f64(out, dtype), want, dtype, "decode step")


def test_out_of_pool_table_entry_is_contained():
    """An entry naming a block outside the pool is never dereferenced (no fault); other rows
    are unaffected bit for bit. With PKV_CHECK=1 the call is refused before launching."""
    m = pkv()
    rng = np.random.default_rng(11)
    p = H.random_problem(rng, [40, 300, 77], 4, 4, 128, "f16")
    d = G.device_problem(p)
    ref = W.to_storage_numpy(run_decode(p, d, 0.1), "f16")
    bad = p["tables"].copy()
    bad[1, 3] = p["nb"] + 1000
    d_bad = dict(d, tables=torch.from_numpy(bad).cuda())
    got = W.to_storage_numpy(run_decode(p, d_bad, 0.1), "f16")
    np.testing.assert_array_equal(got[[0, 2]].view(np.uint8), ref[[0, 2]].view(np.uint8))
    assert np.all(np.isfinite(got[1].astype(np.float32)))
    os.environ["PKV_CHECK"] = "1"
    try:
        with pytest.raises(m.PkvError) as e:
            run_decode(p, d_bad, 0.1)
        assert e.value.status == 7
        run_decode(p, d, 0.1)  # a valid table passes the check
    finally:
        del os.environ["PKV_CHECK"]


# ---- full-size workloads, in the configuration the benchmark times ----------------------

FULL = ["llama2_7b", "qwen25_7b", "prefix_shared", "long_context"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    m = pkv()
    shape = W.SHAPES[name]
    print(f"[full] {name}", flush=True)
    fp = G.full_size_problem(shape)
    scale = G.scale_for(shape.hd)
    out = m.pkv_decode_attn(fp["q"], fp["k_cache"], fp["v_cache"],
                            torch.from_numpy(fp["tables"]).cuda(),
                            torch.from_numpy(fp["lens"]).cuda(), num_kv_heads=shape.Hkv,
                            scale=scale, max_context_len=fp["max_ctx"])
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    rows = G.sample_rows(fp["lens"], 6, np.random.default_rng(shape.seed))
    want = G.sampled_oracle(fp, rows, scale)
    got = G.gpu_f64(out[rows], shape.dtype)
    G.assert_close(got, want, shape.dtype, f"{name} rows {rows}")


@pytest.mark.parametrize("dtype,hq,hkv,kernel", [("bf16", 4, 4, 0), ("bf16", 8, 2, 0),
                                                 ("f16", 8, 2, 1), ("f32", 2, 2, 0)])
def test_shared_block_mark_changes_nothing(dtype, hq, hkv, kernel):
    """Entries marked as shared blocks (only the loads' cache policy differs) give the same
    bits as the unmarked table, through the plain and the fused-append paths, and pass the
    PKV_CHECK index validation."""
    m = pkv()
    rng = np.random.default_rng(12)
    lens = [37, 512, 700, 1300, 16]
    base = H.random_problem(rng, lens, hq, hkv, 128, dtype, nb=400)
    seq_k = [x.copy() for x in base["seq_k"]]
    seq_v = [x.copy() for x in base["seq_v"]]
    for i in (2, 3):  # sequences 1..3 share sequence 1's first 32 blocks
        seq_k[i][:512] = seq_k[1][:512]
        seq_v[i][:512] = seq_v[1][:512]
    tables = base["tables"].copy()
    for i in (2, 3):
        tables[i, :32] = tables[1, :32]
    k, v = H.build_caches(seq_k, seq_v, tables, lens, 400, hkv, 128, 16, dtype)
    p = dict(base, seq_k=seq_k, seq_v=seq_v, tables=tables, k_cache=k, v_cache=v)
    marked = tables.copy()
    marked[1:4, :32] |= m.BLOCK_SHARED
    pm = dict(p, tables=marked)
    out = W.to_storage_numpy(run_decode(p, G.device_problem(p), 0.1, kernel), dtype)
    out_m = W.to_storage_numpy(run_decode(pm, G.device_problem(pm), 0.1, kernel), dtype)
    np.testing.assert_array_equal(out.view(np.uint8), out_m.view(np.uint8))
    G.assert_close(H.f64(out, dtype), G.oracle_out(p, 0.1), dtype, "shared prefix")
    os.environ["PKV_CHECK"] = "1"
    try:
        run_decode(pm, G.device_problem(pm), 0.1, kernel)
    finally:
        del os.environ["PKV_CHECK"]
    # fused append with the marked table: the newest tokens are in private blocks
    B = len(lens)
    k_new = W.normal_values(rng, (B, hkv, 128), dtype)
    v_new = W.normal_values(rng, (B, hkv, 128), dtype)
    res = []
    for tb in (tables, marked):
        d = G.device_problem(dict(p, tables=tb))
        prev = m.pkv_set_attn_kernel(kernel)
        try:
            o = m.pkv_decode_append_attn(d["q"], G.to_dev(k_new, dtype), G.to_dev(v_new, dtype),
                                         d["k_cache"], d["v_cache"], d["tables"], d["lens"],
                                         num_kv_heads=hkv, scale=0.1,
                                         max_context_len=G.max_context(lens))
            torch.cuda.synchronize()
        finally:
            m.pkv_set_attn_kernel(prev)
        res.append((W.to_storage_numpy(o, dtype).view(np.uint8),
                    W.to_storage_numpy(d["k_cache"], dtype).reshape(-1).view(np.uint8),
                    W.to_storage_numpy(d["v_cache"], dtype).reshape(-1).view(np.uint8)))
    for a_, b_ in zip(*res):
        np.testing.assert_array_equal(a_, b_)
