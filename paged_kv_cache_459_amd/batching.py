"""Continuous batching over the paged cache: the decode step loop.

[P1] §四 "連續批次": requests leave the batch as soon as they are done and new ones join at any
step; the paged cache allows it because blocks are taken on demand and released per request
([P1] §三 步驟一..四). Admission rule (ours; the pages give none, and leave preemption to
vLLM's tuning, so the rule never needs it):

* waiting requests are served first-come first-served, never reordered;
* a step is: (1) retire the running requests that produced their max new tokens (their
  blocks go back to the pool); (2) admit queue heads that have arrived while fewer than
  ``max_batch`` run and the free blocks cover the head's final size (prompt + max new tokens)
  on top of what the running requests may still take; an admitted request's prompt slots are
  allocated and its prompt K/V written (``pkv_write``), and, if the caller asks
  (``prefill``), the written prompt tokens are attended causally (``pkv_prefill_attn``, the
  cached prefix included); (3) decode: every running request, in
  admission order, appends one token, whose K/V are stored and attended to in the fused
  decode step (``pkv_decode_append_stream`` + ``pkv_decode_append_merge``).

With ``prefix_cache=True`` requests carry their prompt's token ids and admission starts each
sequence with ``add_seq_tokens`` (automatic prefix caching, [P1] §五 / §八, [P3] §4.2): the
prompt's cached full blocks are shared and only the tokens after them are written; decode
appends with the new tokens' ids so that filled blocks are indexed too. Tables are exported
with shared blocks marked, so the attention kernels keep those in the L2.

Host bookkeeping only: the allocator is the library's C++ allocator and every device step
runs in the library's kernels. Host buffers for tables and slots are pinned and
double-buffered, so the host may prepare the next step while the current one runs.
"""

import math

import numpy as np
import torch

from . import api
from .api import BLOCK_SIZE, BlockAllocator


def _blocks(n):
    return -(-np.asarray(n, dtype=np.int64) // BLOCK_SIZE)


class ContinuousBatch:
    def __init__(self, k_cache, v_cache, *, num_q_heads, num_kv_heads, head_dim, max_batch,
                 max_context_len, free_order=None, prefix_cache=False):
        self.k_cache, self.v_cache = k_cache, v_cache
        self.prefix_cache = bool(prefix_cache)
        self.Hq, self.Hkv, self.hd = num_q_heads, num_kv_heads, head_dim
        self.dtype = k_cache.dtype
        self.device = k_cache.device
        self.nb = api._num_blocks(k_cache, num_kv_heads, head_dim)
        self.alloc = BlockAllocator(self.nb, BLOCK_SIZE, free_order)
        self.max_batch = int(max_batch)
        self.max_ctx = int(max_context_len)
        self.max_blocks = int(_blocks(self.max_ctx))
        # waiting queue (arrival order) and running requests (admission order)
        self.queue = []
        self.run_id = np.zeros(0, np.int64)
        self.run_final = np.zeros(0, np.int64)  # prompt + max new tokens
        self.run_new = np.zeros(0, np.int64)    # max new tokens
        self.run_done = np.zeros(0, np.int64)   # tokens produced so far
        self.step_no = 0
        self.prompt_slots = None
        # two sets of step buffers [lens | tables | prompt slots], pinned on the host and on
        # the device; a step fills one set while the previous step's copies may still read
        # the other
        self._slot0 = self.max_batch + self.max_batch * self.max_blocks
        self._plan0 = self._slot0 + self.max_batch * self.max_ctx
        plan_cap = (int(api.lib.pkv_decode_plan_max_ints(self.max_batch, self.max_blocks))
                    if self.prefix_cache else 0)
        n_int = self._plan0 + plan_cap
        self._pin = [torch.empty(n_int, dtype=torch.int32, pin_memory=True) for _ in range(2)]
        self._dev = [torch.empty(n_int, dtype=torch.int32, device=self.device) for _ in range(2)]
        self._free = [torch.cuda.Event() for _ in range(2)]
        self._set = 0
        self._set_ready = False
        self.kernel = api.pkv_decode_kernel(num_q_heads, num_kv_heads, self.dtype)
        self.W = api.pkv_decode_num_workers(num_q_heads, num_kv_heads, head_dim, self.dtype)
        ws = api.pkv_decode_stream_workspace_bytes(self.max_batch, num_q_heads, num_kv_heads,
                                                   head_dim, self.dtype, self.W)
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=self.device)

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
        if _blocks(prompt_len + max_new_tokens) > self.nb:
            raise ValueError("request larger than the whole pool")
        ids = None if token_ids is None else np.ascontiguousarray(token_ids, dtype=np.int32)
        self.queue.append((int(rid), int(prompt_len), int(max_new_tokens), int(arrival_step),
                           ids))

    def idle(self):
        return not self.queue and len(self.run_id) == 0

    def running(self):
        return self.run_id.copy()

    # -- phases 1 and 2 --------------------------------------------------------------------
    def _take_set(self):
        """The step's buffer set, once its previous copies have run."""
        if not self._set_ready:
            self._free[self._set].synchronize()
            self._set_ready = True
        return self._set

    def _release_set(self):
        self._free[self._set].record()
        self._set ^= 1
        self._set_ready = False

    def schedule(self):
        """Retire finished requests, admit arrived ones. Returns (retired ids, admitted
        [(id, prompt_len)], number of prompt tokens to write). With prefix caching the tokens
        to write are each admitted prompt's tokens after its cached ones, and
        ``last_cached`` holds the cached counts."""
        finished = self.run_done >= self.run_new
        retired = self.run_id[finished]
        if len(retired):
            self.alloc.free_many(retired)
            keep = ~finished
            self.run_id, self.run_final = self.run_id[keep], self.run_final[keep]
            self.run_new, self.run_done = self.run_new[keep], self.run_done[keep]
        # what the running requests may still take: final blocks minus the blocks they hold
        held = _blocks(self.run_final - self.run_new + self.run_done)
        reserve = int((_blocks(self.run_final) - held).sum())
        admitted, cached = [], []
        T = 0
        while self.queue and self.queue[0][3] <= self.step_no and \
                len(self.run_id) + len(admitted) < self.max_batch:
            rid, p, m, _, ids = self.queue[0]
            need = int(_blocks(p + m))
            if self.alloc.num_free() - reserve < need:
                break
            self.queue.pop(0)
            s = self._take_set()
            pin = self._pin[s].numpy()
            if ids is not None:  # prefix caching: shares the cached full blocks
                slots, c = self.alloc.add_seq_tokens(rid, ids)
                pin[self._slot0 + T:self._slot0 + T + p - c] = slots[c:]
            else:
                c = 0
                self.alloc.add_seq(rid)
                self.alloc.append([rid], [p], slots_out=pin[self._slot0 + T:self._slot0 + T + p])
            T += p - c
            reserve += need - int(_blocks(p))
            admitted.append((rid, p, m))
            cached.append(c)
        self.last_cached = cached
        self.last_admitted = [(a[0], a[1], c) for a, c in zip(admitted, cached)]
        if T:
            s = self._set
            self.prompt_slots = self._dev[s][self._slot0:self._slot0 + T]
            self.prompt_slots.copy_(self._pin[s][self._slot0:self._slot0 + T], non_blocking=True)
        else:
            self.prompt_slots = None
        if admitted:
            self.run_id = np.concatenate([self.run_id, [a[0] for a in admitted]]).astype(np.int64)
            self.run_final = np.concatenate([self.run_final,
                                             [a[1] + a[2] for a in admitted]]).astype(np.int64)
            self.run_new = np.concatenate([self.run_new, [a[2] for a in admitted]]).astype(np.int64)
            self.run_done = np.concatenate([self.run_done, np.zeros(len(admitted), np.int64)])
        return retired, [(a[0], a[1]) for a in admitted], T

    def write_prompts(self, k, v):
        """The admitted prompts' K/V, [T, Hkv, hd] in admission order (T from schedule())."""
        if self.prompt_slots is None:
            if k.shape[0]:
                raise ValueError("no prompt was admitted this step")
            return
        api.pkv_write(k, v, self.k_cache, self.v_cache, self.prompt_slots)

    def prefill(self, q, scale, out=None, events=None):
        """Causal attention of the prompt tokens written this step (after write_prompts, before
        decode): q [T, Hq, hd] in the rows of write_prompts (each admitted prompt's tokens
        after its cached ones) attends over its own prompt, cached prefix included
        (pkv_prefill_attn). Returns out [T, Hq, hd]. ``events``: optional two
        torch.cuda.Events recorded before and after the attention."""
        adm = getattr(self, "last_admitted", [])
        T = sum(p - c for _, p, c in adm)
        if q.shape[0] != T:
            raise ValueError(f"q has {q.shape[0]} rows, the admitted prompts {T} tokens")
        if T == 0:
            return q.new_empty((0, self.Hq, self.hd))
        A, mb = len(adm), self.max_blocks
        if not hasattr(self, "_pf_pin"):  # two pinned/device sets: tables, lengths, plan
            tmax = self.max_batch * self.max_ctx
            cap = (16 + 3 * tmax + 1 +
                   8 * tmax * max(1, -(-mb // api.PREFILL_MAX_BLOCKS)))
            self._pf_n = self.max_batch * mb + 2 * self.max_batch + 1
            n = self._pf_n + cap
            self._pf_pin = [torch.empty(n, dtype=torch.int32, pin_memory=True) for _ in range(2)]
            self._pf_dev = [torch.empty(n, dtype=torch.int32, device=self.device)
                            for _ in range(2)]
            self._pf_free = [torch.cuda.Event() for _ in range(2)]
            self._pf_set = 0
            self._pf_ws = None
        s = self._pf_set
        self._pf_free[s].synchronize()  # the copies that last read this set have run
        pin = self._pf_pin[s].numpy()
        tab = pin[:A * mb].reshape(A, mb)
        o = self.max_batch * mb
        lens = pin[o:o + A]
        qs = pin[o + self.max_batch:o + self.max_batch + A + 1]
        self.alloc.tables(np.array([a[0] for a in adm], np.int64), mb, tables_out=tab,
                          lens_out=lens, mark_shared=True)
        qs[0] = 0
        qs[1:] = np.cumsum([p - c for _, p, c in adm])
        plan = api.pkv_prefill_plan(qs, lens, num_q_heads=self.Hq, num_kv_heads=self.Hkv,
                                    max_blocks=mb, max_context_len=self.max_ctx,
                                    dtype=self.dtype, out=pin[self._pf_n:])
        if plan.ctypes.data != pin[self._pf_n:].ctypes.data:
            raise RuntimeError("prefill plan larger than its pinned buffer")
        dev = self._pf_dev[s]
        dev[:A * mb].copy_(self._pf_pin[s][:A * mb], non_blocking=True)
        end = self._pf_n + len(plan)
        dev[self._pf_n:end].copy_(self._pf_pin[s][self._pf_n:end], non_blocking=True)
        self._pf_free[s].record()
        self._pf_set ^= 1
        need = api.pkv_prefill_workspace_bytes(self.Hq, self.Hkv, self.hd, plan)
        if need and (self._pf_ws is None or self._pf_ws.numel() < need):
            self._pf_ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        if events is not None:
            events[0].record()
        out = api.pkv_prefill_attn(q, self.k_cache, self.v_cache, dev[:A * mb].view(A, mb),
                                   plan, dev[self._pf_n:end], num_kv_heads=self.Hkv,
                                   scale=scale, max_context_len=self.max_ctx,
                                   workspace=self._pf_ws if need else None, out=out)
        if events is not None:
            events[1].record()
        self.last_prefill_tables = tab.copy()
        return out

    # -- phase 3 ---------------------------------------------------------------------------
    def decode(self, q, k_new, v_new, scale, out=None, events=None, new_ids=None):
        """One decode step of every running request (rows of q/k_new/v_new in admission
        order; new_ids: the new tokens' ids, with prefix caching). Returns out [B, Hq, hd].
        ``events``: optional torch.cuda.Events: three (before the first kernel, after the stream
        pass, after the merge) or four (before, after the shared pass, after the stream pass,
        after the merge; with prefix caching the step runs a shared-prefix plan)."""
        if (new_ids is not None) != self.prefix_cache:
            raise ValueError("new_ids are given exactly when prefix caching is on")
        B = len(self.run_id)
        self.step_no += 1
        if B == 0:
            if self._set_ready:
                self._release_set()
            return q.new_empty((0, self.Hq, self.hd))
        s = self._take_set()
        flat = self._pin[s].numpy()
        lens_h = flat[:B]
        tables_h = flat[self.max_batch:self.max_batch + B * self.max_blocks].reshape(
            B, self.max_blocks)
        self.alloc.append(self.run_id, np.ones(B, np.int32), want_slots=False,
                          token_ids=new_ids)
        self.alloc.tables(self.run_id, self.max_blocks, tables_out=tables_h, lens_out=lens_h,
                          mark_shared=True)
        self.run_done += 1
        dev = self._dev[s]
        nt = self.max_batch + B * self.max_blocks
        dev[:B].copy_(self._pin[s][:B], non_blocking=True)
        dev[self.max_batch:nt].copy_(self._pin[s][self.max_batch:nt], non_blocking=True)
        plan = plan_d = None
        self.last_plan_units = 0
        if self.prefix_cache:  # requests share cached blocks: a shared-prefix plan
            plan = api.pkv_decode_plan(tables_h, lens_h, num_q_heads=self.Hq,
                                       num_kv_heads=self.Hkv, num_blocks=self.nb,
                                       max_context_len=self.max_ctx, dtype=self.dtype,
                                       out=flat[self._plan0:])
            self.last_plan_units = int(plan[4])
            plan_d = dev[self._plan0:self._plan0 + len(plan)]
            plan_d.copy_(self._pin[s][self._plan0:self._plan0 + len(plan)], non_blocking=True)
            need = api.pkv_decode_planned_workspace_bytes(B, self.Hq, self.Hkv, self.hd,
                                                          self.dtype, self.W, plan)
            if need > self.workspace.numel():
                self.workspace = torch.empty(need, dtype=torch.uint8, device=self.device)
        self._release_set()
        lens_d = dev[:B]
        tables_d = dev[self.max_batch:self.max_batch + B * self.max_blocks].view(
            B, self.max_blocks)
        if out is None:
            out = torch.empty_like(q)
        if events is not None:
            events[0].record()
        if plan is not None:  # shared pass, stream pass, merge
            ev = None if events is None else ([events[1], events[1], events[2]]
                                              if len(events) == 3 else events[1:4])
            api.pkv_decode_planned(q, self.k_cache, self.v_cache, tables_d, lens_d, plan, plan_d,
                                   num_kv_heads=self.Hkv, scale=scale,
                                   max_context_len=self.max_ctx, num_workers=self.W,
                                   workspace=self.workspace, k_new=k_new, v_new=v_new, out=out,
                                   events=ev)
        else:
            if events is not None and len(events) == 4:
                events[1].record()  # no shared pass
            api.pkv_decode_append_stream(q, k_new, v_new, self.k_cache, self.v_cache, tables_d,
                                         lens_d, num_kv_heads=self.Hkv, scale=scale,
                                         max_context_len=self.max_ctx, num_workers=self.W,
                                         workspace=self.workspace, out=out)
            if events is not None:
                events[-2].record()
            api.pkv_decode_append_merge(out, k_new, v_new, self.k_cache, self.v_cache, tables_d,
                                        lens_d, self.workspace, num_kv_heads=self.Hkv,
                                        max_context_len=self.max_ctx, num_workers=self.W)
            if events is not None:
                events[-1].record()
        self.last_tables = tables_h
        self.last_lens = lens_h
        return out

    def usage(self):
        return self.alloc.usage()

    def close(self):
        self.alloc.close()


def default_scale(head_dim):
    return 1.0 / math.sqrt(head_dim)
