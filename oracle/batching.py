"""Continuous batching over the paged cache: the step loop, in float64 / plain Python.

Test infrastructure only (see the package docstring).

[P1] §四 "連續批次": a request leaves the batch as soon as it is done and new requests join
at any step, which the paged cache makes possible because blocks are taken when a request
needs them and released on their own when it finishes ([P1] §三 步驟一..四). The pages give
no admission rule; ours (the plain reading that never needs preemption, which the pages
leave to vLLM's tuning):

* a request is (id, prompt length, max new tokens, arrival step); the waiting queue is
  first-come first-served and is never reordered;
* a step has three phases:
  1. retire: every running request that has produced its max new tokens is freed, in
     running order ([P1] §三 步驟四);
  2. admit: while the queue's head has arrived, fewer than ``max_batch`` requests run, and
     the free blocks cover the head's final size (prompt + max new tokens, in blocks) on top
     of what the running requests may still take before they finish, the head joins: its
     sequence is created, its prompt's slots are allocated and its prompt K/V written
     ([P1] §三 步驟一..二); optionally (``prefill``) the written prompt tokens are then
     attended, causally. The first head that does not fit stops admission for the step;
  3. decode: every running request, in admission order, appends one token: its K/V are
     written into the slot the allocator gives and attention runs over all of its tokens
     ([P1] §三 步驟三).

With ``prefix_cache`` the requests carry their prompt's token ids: admission starts each
sequence with ``add_seq_tokens`` (automatic prefix caching: the prompt's cached full blocks
are shared and only the rest of the prompt is written) and decode appends with the new
tokens' ids. The admission test is unchanged (a hit is not counted on).
"""

import numpy as np

from . import attention, cache_write
from .allocator import BlockAllocator


def blocks_for(n, bs):
    return -(-int(n) // bs)


class Request:
    def __init__(self, rid, prompt_len, max_new, arrival, token_ids=None):
        self.rid, self.prompt_len, self.max_new, self.arrival = rid, prompt_len, max_new, arrival
        self.token_ids = token_ids
        self.generated = 0
        self.cached = 0


class BatchingLoop:
    def __init__(self, num_blocks, bs, hkv, hd, dtype, *, max_batch, free_order=None,
                 storage_dtype=None, nan_fill=None, prefix_cache=False):
        self.prefix_cache = prefix_cache
        self.alloc = BlockAllocator(num_blocks, bs, free_order)
        self.bs, self.hkv, self.hd, self.dtype = bs, hkv, hd, dtype
        self.max_batch = max_batch
        size = num_blocks * hkv * hd * bs
        self.k_cache = np.full(size, nan_fill, storage_dtype)
        self.v_cache = np.full(size, nan_fill, storage_dtype)
        self.queue = []     # waiting requests, arrival order
        self.running = []   # admitted requests, admission order
        self.step_no = 0

    def submit(self, rid, prompt_len, max_new, arrival, token_ids=None):
        assert prompt_len >= 1 and max_new >= 1
        assert (token_ids is not None) == self.prefix_cache
        assert token_ids is None or len(token_ids) == prompt_len
        self.queue.append(Request(rid, prompt_len, max_new, arrival, token_ids))

    def _future_blocks(self):
        """Blocks the running requests may still take before they finish."""
        total = 0
        for r in self.running:
            n = self.alloc.seq_len(r.rid)
            total += blocks_for(r.prompt_len + r.max_new, self.bs) - blocks_for(n, self.bs)
        return total

    def schedule(self):
        """Phases 1 and 2. Returns (retired ids, admitted requests, slots of the prompt tokens
        to write, in admission order: with prefix caching, each request's tokens after its
        cached ones)."""
        retired = [r.rid for r in self.running if r.generated == r.max_new]
        for rid in retired:
            self.alloc.free_seq(rid)
        self.running = [r for r in self.running if r.generated < r.max_new]
        admitted, slots = [], []
        while self.queue and self.queue[0].arrival <= self.step_no and \
                len(self.running) < self.max_batch:
            head = self.queue[0]
            need = blocks_for(head.prompt_len + head.max_new, self.bs)
            if self.alloc.num_free() - self._future_blocks() < need:
                break
            self.queue.pop(0)
            if self.prefix_cache:
                s, head.cached = self.alloc.add_seq_tokens(head.rid, head.token_ids)
                slots.extend(s[head.cached:])
            else:
                self.alloc.add_seq(head.rid)
                s, _ = self.alloc.append([head.rid], [head.prompt_len])
                slots.extend(s)
            self.running.append(head)
            admitted.append(head)
        return retired, admitted, np.asarray(slots, np.int32)

    def write_prompts(self, k, v, slots):
        """Phase 2's write: k, v [T, Hkv, hd] storage arrays for the admitted prompts."""
        self.k_cache, self.v_cache = cache_write.write_kv(
            k, v, self.k_cache, self.v_cache, slots, hkv=self.hkv, hd=self.hd, bs=self.bs,
            dtype=self.dtype)

    def prefill(self, q, admitted, scale):
        """Phase 2's attention, after the write: the admitted prompts' written tokens (each
        prompt's tokens after its cached ones), q [T, Hq, hd] in admission order, attend
        causally over their own prompts ([P1] §三 步驟二; the causal reading of
        attention.prefill_attention). Returns float64 [T, Hq, hd]."""
        if not admitted:
            return np.zeros((0,) + np.shape(q)[1:])
        ids = [a.rid for a in admitted]
        mb = max(len(self.alloc.blocks[i]) for i in ids)
        tables, lens = self.alloc.tables(ids, mb)
        tables = np.asarray(tables, np.int32).reshape(len(ids), mb)
        qs = np.concatenate([[0], np.cumsum([a.prompt_len - a.cached for a in admitted])])
        return attention.prefill_attention(q, self.k_cache, self.v_cache, tables,
                                           np.asarray(lens, np.int32), qs.astype(np.int32),
                                           scale=scale, hkv=self.hkv, hd=self.hd, bs=self.bs,
                                           dtype=self.dtype)

    def decode(self, q, k_new, v_new, scale, new_ids=None):
        """Phase 3 for the running requests (admission order); new_ids: the new tokens' ids
        (prefix caching). Returns (out float64 [B, Hq, hd], the step's slots, tables,
        lengths)."""
        ids = [r.rid for r in self.running]
        if not ids:  # nothing runs this step
            self.step_no += 1
            return (np.zeros((0,) + np.shape(q)[1:]), np.zeros(0, np.int32),
                    np.zeros((0, 1), np.int32), np.zeros(0, np.int32))
        if self.prefix_cache:
            slots, cows = self.alloc.append_tokens(ids, [1] * len(ids), list(new_ids))
        else:
            slots, cows = self.alloc.append(ids, [1] * len(ids))
        assert not cows  # appends never land in a shared block (only full blocks are shared)
        self.k_cache, self.v_cache = cache_write.write_kv(
            k_new, v_new, self.k_cache, self.v_cache, np.asarray(slots, np.int32),
            hkv=self.hkv, hd=self.hd, bs=self.bs, dtype=self.dtype)
        mb = max([1] + [len(self.alloc.blocks[i]) for i in ids])
        tables, lens = self.alloc.tables(ids, mb)
        tables = np.asarray(tables, np.int32).reshape(len(ids), mb)
        lens = np.asarray(lens, np.int32)
        out = attention.decode_attention(q, self.k_cache, self.v_cache, tables, lens,
                                         scale=scale, hkv=self.hkv, hd=self.hd, bs=self.bs,
                                         dtype=self.dtype)
        for r in self.running:
            r.generated += 1
        self.step_no += 1
        return out, np.asarray(slots, np.int32), tables, lens

    def idle(self):
        return not self.queue and not self.running
