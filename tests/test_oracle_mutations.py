"""Plant plausible mistakes in the oracle (on the CPU) and check that its pins catch them.

Each case patches one oracle function with a wrong variant (a dropped scale, a wrong
kv-head mapping, an off-by-one gather, a transposed tile, an unweighted merge, a LIFO free
list, a missing copy-on-write, a skipped, reversed or half block copy, shared blocks counted per owner, a reservation
counted as used, admission without headroom or out of arrival order, a prefix block matched without its
parent, a prefill without its causal mask or off by one) and runs an existing pin, which must then fail.
"""

import numpy as np
import pytest

from oracle import allocator as AL
from oracle import attention as A
from oracle import batching as OB
from oracle import cache_write as CW
from oracle import layout as L
from oracle import utilisation as U
from tests import test_oracle_allocator as TAL
from tests import test_oracle_attention as TA
from tests import test_oracle_batching as TOB
from tests import test_oracle_beam as TB
from tests import test_oracle_prefill as TPF
from tests import test_oracle_prefix_cache as TPC
from tests import test_oracle_utilisation as TU


def _fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_dropped_scale_is_caught(monkeypatch):
    orig = A._dense_attention_one
    monkeypatch.setattr(A, "_dense_attention_one", lambda q, K, V, scale: orig(q, K, V, 1.0))
    _fails(TA.test_matches_torch_sdpa, "f32", 2, 2)


def test_wrong_gqa_head_mapping_is_caught(monkeypatch):
    def bad(q, k_cache, v_cache, block_tables, context_lens, *, scale, hkv, hd, bs, dtype,
            num_blocks=None):
        qf = L.to_f64(q, dtype)
        B, hq, _ = qf.shape
        out = np.zeros((B, hq, hd))
        nbk = np.asarray(k_cache).size // (hkv * hd * bs)
        for i in range(B):
            n = int(context_lens[i])
            if n == 0:
                continue
            K, V = A.gather_sequence(k_cache, v_cache, block_tables[i], n, num_blocks=nbk,
                                     hkv=hkv, hd=hd, bs=bs, dtype=dtype)
            for h in range(hq):
                g = h % hkv  # wrong: interleaved instead of contiguous groups
                out[i, h] = A._dense_attention_one(qf[i, h], K[:, g], V[:, g], scale)
        return out
    monkeypatch.setattr(A, "decode_attention", bad)
    _fails(TA.test_matches_torch_sdpa, "f32", 8, 2)


def test_off_by_one_gather_is_caught(monkeypatch):
    orig = A.gather_sequence

    def short(k_cache, v_cache, row, n, **kw):
        K, V = orig(k_cache, v_cache, row, n, **kw)
        if n > 1:
            K[-1], V[-1] = K[-2], V[-2]  # last token read from the wrong slot
        return K, V
    monkeypatch.setattr(A, "gather_sequence", short)
    _fails(TA.test_hand_example)


def test_transposed_tile_is_caught(monkeypatch):
    def bad_k(k_cache, block, hkv, hd, bs, dtype):
        x = L.chunk_elems(dtype)
        tile = np.asarray(k_cache).reshape(-1, hkv, bs, hd // x, x)[block]  # token-major: wrong
        return tile.transpose(1, 0, 2, 3).reshape(bs, hkv, hd)
    monkeypatch.setattr(L, "k_tile_tokens", bad_k)
    _fails(TA.test_layout_reading_matches_header_formula, "f16")


def test_unweighted_merge_is_caught(monkeypatch):
    def bad(m, l, o):
        return np.asarray(o).sum(0) / np.asarray(l).sum()
    monkeypatch.setattr(A, "merge_partials", bad)
    _fails(TA.test_partition_merge_equals_unsplit, 32)


def test_lifo_free_list_is_caught(monkeypatch):
    orig_free = AL.BlockAllocator.free_seq

    def lifo_free(self, seq):
        before = list(self.free)
        orig_free(self, seq)
        new = list(self.free)[len(before):]
        self.free = AL.deque(list(reversed(new)) + before)
    monkeypatch.setattr(AL.BlockAllocator, "free_seq", lifo_free)
    _fails(TAL.test_p1_shared_blocks_example)


def test_missing_copy_on_write_is_caught(monkeypatch):
    monkeypatch.setattr(AL.BlockAllocator, "_needs",
                        lambda self, seq, ntok: (False, -(-(self.length[seq] + ntok) // self.bs)
                                                 - -(-self.length[seq] // self.bs)))
    _fails(TAL.test_copy_on_write_pair_reported)


def test_skipped_block_copy_is_caught(monkeypatch):
    monkeypatch.setattr(CW, "copy_blocks",
                        lambda kc, vc, pairs, **kw: (np.array(kc, copy=True),
                                                     np.array(vc, copy=True)))
    _fails(TB.test_beam_loop_keeps_every_beams_history, "f32")


def test_reversed_block_copy_is_caught(monkeypatch):
    orig = CW.copy_blocks
    monkeypatch.setattr(CW, "copy_blocks",
                        lambda kc, vc, pairs, **kw: orig(kc, vc, [(d, s) for s, d in pairs], **kw))
    _fails(TB.test_beam_loop_keeps_every_beams_history, "f32")


def test_copy_of_one_cache_only_is_caught(monkeypatch):
    orig = CW.copy_blocks

    def k_only(kc, vc, pairs, **kw):
        k2, _ = orig(kc, vc, pairs, **kw)
        return k2, np.array(vc, copy=True)
    monkeypatch.setattr(CW, "copy_blocks", k_only)
    _fails(TB.test_beam_loop_keeps_every_beams_history, "bf16")


def test_shared_block_counted_per_owner_is_caught(monkeypatch):
    def per_owner(tables, lengths, bs):
        slots = sum(int(n) for n in lengths)
        blocks = sum(-(-int(n) // bs) for n in lengths)
        return dict(sequences=len(lengths), logical_tokens=slots, blocks_in_use=blocks,
                    slots_filled=slots, utilisation=slots / (blocks * bs) if blocks else 0.0)
    monkeypatch.setattr(U, "paged_usage", per_owner)
    _fails(TU.test_shared_blocks_counted_once)


def test_whole_reservation_counted_as_used_is_caught(monkeypatch):
    monkeypatch.setattr(U, "contiguous_usage",
                        lambda lengths, max_len: (len(lengths) * max_len,) * 2 + (1.0,))
    _fails(TU.test_pages_worked_examples)


def test_admission_without_headroom_is_caught(monkeypatch):
    monkeypatch.setattr(OB.BatchingLoop, "_future_blocks", lambda self: 0)
    with pytest.raises((AssertionError, AL.AllocError)):
        TOB.test_loop_follows_its_rules(12, 4)


def test_admission_out_of_order_is_caught(monkeypatch):
    orig = OB.BatchingLoop.schedule

    def lifo(self):
        self.queue.sort(key=lambda r: (r.arrival > self.step_no, -r.rid))  # newest first
        return orig(self)
    monkeypatch.setattr(OB.BatchingLoop, "schedule", lifo)
    _fails(TOB.test_loop_follows_its_rules, 40, 8)


def test_prefix_match_without_parent_is_caught(monkeypatch):
    """Index blocks by their own ids only (the parent dropped from the key)."""
    class Parentless(dict):
        def _k(self, key):
            return (0, key[1])

        def __getitem__(self, key):
            return dict.__getitem__(self, self._k(key))

        def __setitem__(self, key, value):
            dict.__setitem__(self, self._k(key), value)

        def __delitem__(self, key):
            dict.__delitem__(self, self._k(key))

        def __contains__(self, key):
            return dict.__contains__(self, self._k(key))

        def get(self, key, default=None):
            return dict.get(self, self._k(key), default)
    orig = AL.BlockAllocator.__init__

    def init(self, *a, **kw):
        orig(self, *a, **kw)
        self.index = Parentless()
    monkeypatch.setattr(AL.BlockAllocator, "__init__", init)
    _fails(TPC.test_shared_blocks_hold_each_sequences_own_kv)


def _prefill_with_window(monkeypatch, window):
    """Replace the oracle's prefill by one whose query at position p sees tokens
    [0, window(p, n)) instead of [0, p + 1)."""
    def bad(q, k_cache, v_cache, block_tables, context_lens, query_start, *, scale, hkv, hd,
            bs, dtype, num_blocks=None):
        qf = L.to_f64(q, dtype)
        T, hq, _ = qf.shape
        G = hq // hkv
        nbk = np.asarray(k_cache).size // (hkv * hd * bs)
        out = np.zeros((T, hq, hd))
        qs = [int(x) for x in query_start]
        for i in range(len(qs) - 1):
            n, t = int(context_lens[i]), qs[i + 1] - qs[i]
            if t == 0:
                continue
            K, V = A.gather_sequence(k_cache, v_cache, block_tables[i], n, num_blocks=nbk,
                                     hkv=hkv, hd=hd, bs=bs, dtype=dtype)
            for k in range(t):
                e = max(1, window(n - t + k, n))
                for h in range(hq):
                    out[qs[i] + k, h] = A._dense_attention_one(qf[qs[i] + k, h], K[:e, h // G],
                                                               V[:e, h // G], scale)
        return out
    monkeypatch.setattr(A, "prefill_attention", bad)


def test_prefill_without_causal_mask_is_caught(monkeypatch):
    _prefill_with_window(monkeypatch, lambda p, n: n)
    _fails(TPF.test_first_token_returns_its_value_and_last_equals_decode, "f32", 2, 2)


def test_prefill_causal_off_by_one_is_caught(monkeypatch):
    _prefill_with_window(monkeypatch, lambda p, n: p)
    _fails(TPF.test_brute_force_tiny)
