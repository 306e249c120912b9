"""Continuous batching over the paged cache: the decode step loop.

[P1] §四 "連續批次": requests leave the batch as soon as they are done and new ones join at any
step; the paged cache allows it because blocks are taken on demand and released per request
([P1] §三 步驟一..四). Admission rule (ours; the pages give none, and leave preemption to
vLLM's tuning, so the rule never needs it):

* waiting requests are served first-come first-served, never reordered;
* a step is: (1) retire the running requests that produced their max new tokens (their
  blocks go back to the pool); (2) admit queue heads that have arrived while fewer than
  ``max_batch`` run, the head's whole prompt fits in the step's prompt rows, and the free
  blocks cover the head's final size (prompt + max new tokens) on top of what the running
  requests may still take; an admitted request's prompt slots are allocated and its prompt
  K/V written (``pkv_write``), and, if the caller gives prompt queries, the written prompt
  tokens are attended causally (``pkv_prefill_attn``, the cached prefix included); (3)
  decode: every running request, in admission order, appends one token, whose K/V are
  stored and attended to in the fused decode step.

With ``prefix_cache=True`` requests carry their prompt's token ids and admission starts each
sequence with ``add_seq_tokens`` (automatic prefix caching, [P1] §五 / §八, [P3] §4.2): the
prompt's cached full blocks are shared and only the tokens after them are written; decode
appends with the new tokens' ids so that filled blocks are indexed too, and each step runs
with a shared-prefix plan, which reads the blocks the requests share once.

The whole step is one call into the library's C++ engine (``pkv_engine_step``): the queue,
the running set, the allocator and the pinned, double-buffered staging of tables and slots
live there, and the host prepares the next step while the device runs the current one. This
class only checks and marshals arguments.
"""

import math

import numpy as np

from . import api
from .api import BLOCK_SIZE, BlockAllocator, Engine


class ContinuousBatch:
    def __init__(self, k_cache, v_cache, *, num_q_heads, num_kv_heads, head_dim, max_batch,
                 max_context_len, free_order=None, prefix_cache=False):
        self.prefix_cache = bool(prefix_cache)
        self.Hq, self.Hkv, self.hd = num_q_heads, num_kv_heads, head_dim
        self.nb = api._num_blocks(k_cache, num_kv_heads, head_dim)
        self.max_batch = int(max_batch)
        self.max_ctx = int(max_context_len)
        self.alloc = BlockAllocator(self.nb, BLOCK_SIZE, free_order)
        self.engine = Engine(self.alloc, k_cache, v_cache, num_q_heads=num_q_heads,
                             num_kv_heads=num_kv_heads, head_dim=head_dim,
                             max_batch=max_batch, max_context_len=max_context_len,
                             plan=self.prefix_cache)
        self.kernel = api.pkv_decode_kernel(num_q_heads, num_kv_heads, k_cache.dtype)
        self.W = api.pkv_decode_num_workers(num_q_heads, num_kv_heads, head_dim, k_cache.dtype)

    # -- requests --------------------------------------------------------------------------
    def submit(self, rid, prompt_len, max_new_tokens, arrival_step=0, token_ids=None):
        if (token_ids is not None) != self.prefix_cache:
            raise ValueError("token_ids are given exactly when prefix caching is on")
        if token_ids is not None and len(token_ids) != prompt_len:
            raise ValueError("token_ids must hold prompt_len ids")
        if prompt_len < 1 or max_new_tokens < 1:
            raise ValueError("a request needs a prompt and at least one new token")
        if prompt_len + max_new_tokens > self.max_ctx:
            raise ValueError("request longer than max_context_len")
        if -(-(prompt_len + max_new_tokens) // BLOCK_SIZE) > self.nb:
            raise ValueError("request larger than the whole pool")
        self.engine.submit(rid, prompt_len, max_new_tokens, arrival_step, token_ids)

    def idle(self):
        return self.engine.queued() == 0 and len(self.engine.running()) == 0

    def running(self):
        return self.engine.running()

    # -- the step --------------------------------------------------------------------------
    def step(self, q, k_new, v_new, out, *, scale, k_prompt=None, v_prompt=None, q_prompt=None,
             prefill_out=None, new_ids=None, events=None):
        """One step (retire, admit + prompt write [+ prefill], decode). q/k_new/v_new/out:
        [max_batch, heads, hd] device buffers whose first B rows are the running requests' in
        admission order; k_prompt/v_prompt (and q_prompt/prefill_out): rows for the admitted
        prompts' tokens to write (each prompt's tokens after its cached ones, in admission
        order); new_ids (prefix caching): the new tokens' ids, first B used. Returns the
        engine's info: B, T, retired, admitted, plan units, copy-on-write pairs, queued,
        step number."""
        if (new_ids is not None) != self.prefix_cache:
            raise ValueError("new_ids are given exactly when prefix caching is on")
        return self.engine.step(q, k_new, v_new, out, scale=scale, k_prompt=k_prompt,
                                v_prompt=v_prompt, q_prompt=q_prompt, prefill_out=prefill_out,
                                new_ids=new_ids, events=events)

    def last(self):
        """The last step's retired ids, admitted (id, prompt_len, cached) triples, prompt
        slots, lengths and marked tables."""
        return self.engine.last()

    def sync(self):
        self.engine.sync()

    def usage(self):
        return self.alloc.usage()

    def close(self):
        self.engine.close()
        self.alloc.close()


def default_scale(head_dim):
    return 1.0 / math.sqrt(head_dim)
