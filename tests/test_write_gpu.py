"""pkv_write on the GPU against the oracle scatter: bit-exact over the whole cache."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import cache_write as CW
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu


def _run(dtype, hd, hkv, nb, T, seed, special=True):
    import paged_kv_cache_459_amd as pkv
    rng = np.random.default_rng(seed)
    size = nb * hkv * hd * 16
    kc = W.normal_values(rng, (size,), dtype)
    vc = W.normal_values(rng, (size,), dtype)
    k = W.normal_values(rng, (T, hkv, hd), dtype)
    v = W.normal_values(rng, (T, hkv, hd), dtype)
    slots = rng.choice(nb * 16, size=T, replace=False).astype(np.int32)
    if special and T >= 3:
        slots[0] = -1  # padding token
        slots[1] = nb * 16 + 3  # outside the pool: skipped
        slots[2] = nb * 16 - 1  # last slot of the pool
    want_k, want_v = CW.write_kv(k, v, kc, vc, slots, hkv=hkv, hd=hd, bs=16, dtype=dtype)
    ks, vs = pkv.cache_shapes(nb, hkv, hd, G.TORCH[dtype])
    dk = G.to_dev(kc, dtype).view(ks)
    dv = G.to_dev(vc, dtype).view(vs)
    pkv.pkv_write(G.to_dev(k, dtype), G.to_dev(v, dtype), dk, dv,
                  torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    got_k = W.to_storage_numpy(dk, dtype).reshape(-1)
    got_v = W.to_storage_numpy(dv, dtype).reshape(-1)
    np.testing.assert_array_equal(got_k.view(np.uint8), want_k.view(np.uint8))
    np.testing.assert_array_equal(got_v.view(np.uint8), want_v.view(np.uint8))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("hd", [64, 128])
def test_write_bit_exact(dtype, hd):
    print(f"[write] dtype={dtype} hd={hd}", flush=True)
    _run(dtype, hd, hkv=3, nb=37, T=200, seed=7 + hd)


def test_write_long_context_step_shape():
    """One new token per sequence for 128 sequences, 8 kv heads, bf16."""
    print("[write] 128 tokens x 8 heads bf16", flush=True)
    _run("bf16", 128, hkv=8, nb=3000, T=128, seed=55, special=False)


def test_write_zero_tokens_is_a_noop():
    import paged_kv_cache_459_amd as pkv
    kc, vc = pkv.alloc_caches(2, 1, 64, torch.float16, fill=1.0)
    k = torch.empty(0, 1, 64, dtype=torch.float16, device="cuda")
    pkv.pkv_write(k, k, kc, vc, torch.empty(0, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert bool((kc == 1).all()) and bool((vc == 1).all())


def test_nan_payload_copied_bitwise():
    import paged_kv_cache_459_amd as pkv
    kc, vc = pkv.alloc_caches(2, 1, 64, torch.bfloat16, fill=0.0)
    k = torch.full((1, 1, 64), 0x7E01, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    v = torch.full((1, 1, 64), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    pkv.pkv_write(k, v, kc, vc, torch.tensor([17], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert int((kc.view(torch.int16) == 0x7E01).sum()) == 64
    assert int((vc.view(torch.int16) == -1).sum()) == 64
