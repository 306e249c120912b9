#!/usr/bin/env python3
"""Benchmark of the paged decode hot path on one MI355X.

One step = one decode step of every sequence in the batch, through the whole path:
  1. allocate on demand: the C++ allocator appends one token per sequence (a fresh block for
     sequences whose last block is full) and returns the new tokens' slots;
  2. bring the block tables (pinned host copy: the entries of the blocks just opened) and
     the lengths up to date and copy them, with the slots, to the device on a copy stream
     (double-buffered, so the copy overlaps the previous step's kernels; the host waits
     for it before launching the kernels, so the compute stream has no cross-stream wait);
  3. + 4. the decode step's two kernels (pkv_decode_append_attn): the stream pass, which
     attends with each sequence's new K/V taken from the step's input rows (every wave
     streams an equal share of the batch's K/V tiles), then the merge pass: the log-sum-exp
     merge of the segments cut between waves, and the stores of the new K/V into their slots.

Beam search (--workload beam_search) replaces step 1 by a beam re-selection: each group's
next beams fork from seeded parents among its current beams (batched fork and free), each
appends one token, and the step's copy-on-write pairs go to the device with the full table
export; the step then runs pkv_copy_blocks on those pairs before the two kernels.

Prints one JSON line: the metric (KV-read GB/s over the timed steps), decode tokens/s per
layer, the roofline figure of the stream kernel (algorithmic bytes / its mean duration,
measured with HIP events on the launch stream) and the oracle's throughput on a bounded
sample of the same workload on the host cores.

    python bench.py [--steps K] [--warmup W] [--workload llama2_7b]
"""

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
METRIC = "paged decode attn: KV-read GB/s and % of HBM peak; decode tokens/s per layer"
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}  # MI355X dense matrix cores, published
PREFILL_METRIC = "paged prefill attn: prompt tokens/s per layer and MFMA TFLOP/s"
WORKLOADS = ("llama2_7b", "qwen25_7b", "prefix_shared", "long_context", "beam_search",
             "continuous_batching", "prefix_cache", "prefill")
DESC = {
    "llama2_7b": "Llama-2-7B-shaped single layer decode: MHA 32 x 128, f16, batch 64, "
                 "context U[128,2048], blocks scattered in a pool of 1.1x need",
    "qwen25_7b": "Qwen2.5-7B-shaped GQA decode: 28 q / 4 kv x 128, bf16, batch 256, context "
                 "lognormal(median 1024, sigma 1) clipped to [16,32768]",
    "prefix_shared": "prefix-shared decode: 128 seqs share a 2000-token prefix (125 blocks, "
                     "refcount 128) + private tails U[16,512], MHA 32 x 128, bf16",
    "long_context": "long-context continuous-batching step: 8 seqs at 32768 + 120 at "
                    "U[64,4096], GQA 32 q / 8 kv x 128, bf16",
    "beam_search": "beam search: 32 groups x 4 beams share a 2000-token prefix, a group's "
                   "beams share its tail U[16,512]; every step re-selects each group's 4 beams "
                   "(seeded parents, forks at unaligned lengths), appends one token per beam "
                   "with copy-on-write of shared partly filled blocks, MHA 32 x 128, bf16",
    "continuous_batching": "continuous batching: Llama-2-7B-shaped layer (MHA 32 x 128, f16), at "
                           "most 64 running, prompts U[64,1024], new tokens U[16,256], a "
                           "backlog of 64 then 0.5 arrivals per step; a pool of 4096 blocks "
                           "(half of 64 contiguous 2048-token reservations); each step retires, "
                           "admits (prompt K/V written), then decodes every running request; "
                           "300 untimed steps reach the steady state before the warm-up",
    "prefix_cache": "continuous batching with automatic prefix caching: Qwen2.5-7B-shaped layer "
                    "(GQA 28 q / 4 kv x 128, bf16), at most 128 running, every prompt is one "
                    "2000-token system prompt + U[16,256] own tokens, new tokens U[16,256], "
                    "a backlog of 128 then 1 arrival per step; admission shares the cached "
                    "system-prompt blocks and writes only the rest; 300 untimed steps first",
    "prefill": "chunked prefill, Llama-2-7B-shaped layer (MHA 32 x 128, f16): 16 sequences, "
               "each a cached prefix of U[0,1536] tokens plus a new chunk of 512 (8192 query "
               "tokens); each step writes the chunk's K/V (pkv_write) and runs causal "
               "attention of the new tokens over the paged cache (pkv_prefill_attn)",
}


class TimingEvent:
    """A HIP event used only for timing, with the record / elapsed_time interface of
    torch.cuda.Event. It is created with hipEventDisableSystemFence: a default event's record
    performs a system-scope fence (cache writeback and invalidation) between the kernels it
    separates, which perturbs the kernels that follow it. The timed loop records several per
    step. Created in the HIP runtime torch has loaded (the one libpkv runs in)."""
    FLAGS = 0x20000000  # hipEventDisableSystemFence; timing stays enabled
    _hip = None

    @classmethod
    def runtime(cls):
        if cls._hip is None:
            with open("/proc/self/maps") as f:
                path = next((ln.split()[-1] for ln in f if "libamdhip64" in ln), None)
            if path is None:
                raise RuntimeError("the HIP runtime is not loaded (import torch first)")
            hip = ctypes.CDLL(path)
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
            cls._hip = hip
        return cls._hip

    def __init__(self):
        self.ev = ctypes.c_void_p()
        err = self.runtime().hipEventCreateWithFlags(ctypes.byref(self.ev), self.FLAGS)
        if err:
            raise RuntimeError(f"hipEventCreateWithFlags failed: error {err}")

    def record(self, stream=None):
        import torch
        if stream is not None:
            handle = stream.cuda_stream
        elif hasattr(torch._C, "_cuda_getCurrentRawStream"):  # no Stream object per record
            handle = torch._C._cuda_getCurrentRawStream(torch.cuda.current_device())
        else:
            handle = torch.cuda.current_stream().cuda_stream
        err = self._hip.hipEventRecord(self.ev, ctypes.c_void_p(handle))
        if err:
            raise RuntimeError(f"hipEventRecord failed: error {err}")

    def synchronize(self):
        """Block the host until the work recorded before this event has completed."""
        err = self._hip.hipEventSynchronize(self.ev)
        if err:
            raise RuntimeError(f"hipEventSynchronize failed: error {err}")

    def elapsed_time(self, end):
        """Milliseconds from this event to `end` (both recorded and completed)."""
        ms = ctypes.c_float()
        err = self._hip.hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev)
        if err:
            raise RuntimeError(f"hipEventElapsedTime failed: error {err}")
        return ms.value

    def __del__(self):
        try:
            if self._hip is not None and self.ev:
                self._hip.hipEventDestroy(self.ev)
        except Exception:  # interpreter shutdown: the runtime may already be gone
            pass


def flush_buffer(torch):
    """1 GiB of device scratch for the cache flush (zeros, so that its sum is finite)."""
    return torch.zeros(1 << 28, dtype=torch.float32, device="cuda")


def flush(scratch):
    """Evicts the batch from the L2s and the last-level cache by reading 1 GiB of other data. A
    read leaves the caches holding clean lines, as other layers' reads would; a write would
    leave up to the cache's size of dirty lines, whose write-back would then land in the timed
    kernels."""
    scratch.sum()


def prime(torch, events):
    """Records every timing event once, outside the timed region: a fresh event's first record
    has cost about a millisecond of host time (the timed step's record then overwrites it)."""
    for e in events:
        e.record()
    torch.cuda.synchronize()


def ms_stats(ms):
    """Mean, median, p10 and p90 of per-launch milliseconds."""
    a = np.asarray(ms, dtype=np.float64)
    return {"mean": round(float(a.mean()), 4), "median": round(float(np.median(a)), 4),
            "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4), "n": int(a.size)}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--event-every", type=int, default=4,
                    help="record the per-kernel timing events on every n-th timed step (each "
                         "event is a marker packet between kernels; the wall-clock step time "
                         "is taken over every step)")
    ap.add_argument("--flush", action="store_true",
                    help="before each timed step, read a 1 GiB scratch buffer (evicts the batch "
                         "from the L2s and the 256 MB last-level cache, leaving clean lines); value "
                         "and ms_per_step then come from the step's kernels' event times instead "
                         "of the wall clock")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama2_7b", choices=WORKLOADS)
    ap.add_argument("--kernel", type=int, default=0, help="0 auto, 1 vector, 2 matrix-core")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="oracle time budget for the CPU baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--driver", choices=("auto", "host", "engine"), default="auto",
                    help="decode workloads: 'engine' runs each step as one pkv_engine_beam_step "
                         "call; 'host' drives it from Python (allocator calls, a side-stream "
                         "table upload the host waits for, launches); 'auto': the engine for "
                         "beam search, the host loop for the fixed batches (where the engine's "
                         "staging kernel costs the device about 5 us per step)")
    ap.add_argument("--no-plan", action="store_true",
                    help="decode batches that share blocks without a shared-prefix plan")
    ap.add_argument("--shared-launch", choices=("auto", "one", "two"), default="auto",
                    help="planned batches: the shared pass and the stream pass as the library "
                         "chooses per step (auto), in one launch, or in two")
    ap.add_argument("--with-prefill", action="store_true",
                    help="batching workloads: each step also runs the admitted prompts' causal "
                         "prefill attention (a full serving step)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--duplicate-prefix", action="store_true",
                    help="prefix_shared only: the duplicated-prefix control, where every "
                         "sequence holds private copies of the prefix blocks (same shapes, "
                         "lengths and contents; no block is shared)")
    args = ap.parse_args()
    if args.duplicate_prefix and args.workload != "prefix_shared":
        ap.error("--duplicate-prefix applies to --workload prefix_shared")
    return args


def kernel_source_digest(workload="llama2_7b"):
    """Digest of the kernel sources a workload's dominant kernel is built from (a change
    there makes its committed counter figures stale)."""
    files = (("pkv_prefill.hip", "pkv_kernels.h") if workload == "prefill"
             else ("pkv_attn.hip", "pkv_kernels.h"))
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "paged_kv_cache_459_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, digest):
    """HBM traffic per launch of the workload's dominant kernel from the committed counter
    summary, if it was taken on the current kernel source; else None."""
    name = "attn_prefill" if workload == "prefill" else f"attn_stream_{workload}"
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_digest") != digest:
        return None
    return rec.get("hbm_bytes_per_launch")


class Workload:
    """Sequences held by the C++ allocator plus device caches filled with seeded values."""

    def __init__(self, name, total_steps, torch, pkv, W, plan=True, duplicate_prefix=False,
                 engine=True, shared_launch="auto"):
        self.name = name
        self.shared_launch = shared_launch
        self.torch = torch
        self.duplicate_prefix = duplicate_prefix and name == "prefix_shared"
        # shared-prefix plans for the batches that share blocks
        self.planned = plan and name in ("prefix_shared", "beam_search") and not self.duplicate_prefix
        self.gen = W  # the seeded input generators
        shape = self.shape = W.SHAPES[name]
        rng = W.rng_for(shape.seed)
        lens = W.draw_lengths(shape, rng)  # lengths after the first step's token
        self.B, self.Hq, self.Hkv, self.hd = shape.B, shape.Hq, shape.Hkv, shape.hd
        self.dt = W.torch_dtype(shape.dtype)
        self.eb = 4 if shape.dtype == "f32" else 2
        nb = W.pool_blocks(lens)
        grow_blocks = sum(W.blocks_for(n + total_steps) - W.blocks_for(n) for n in lens)
        if nb - sum(W.blocks_for(n) for n in lens) < grow_blocks:
            nb += grow_blocks  # keep the run inside the pool
        self.NB = nb
        order = rng.permutation(nb).astype(np.int32)
        self.alloc = pkv.BlockAllocator(nb, 16, order)
        self.seqs = np.arange(self.B, dtype=np.int64)
        self.beam = name == "beam_search"
        self.cows = []  # copy-on-write pairs per timed step
        self.cows_all = []  # and per step of the whole run (warm-up included)
        if self.beam:
            # the prefix, then per group its tail, then the group's beams forked from it (they
            # share every block, the partly filled last one included, until they append)
            parent = 10_000_000
            self.alloc.add_seq(parent)
            self.alloc.append([parent], [W.PREFIX_TOKENS], want_slots=False)
            groups = self.B // W.BEAMS
            roots = np.arange(parent + 1, parent + 1 + groups, dtype=np.int64)
            self.alloc.fork_many(np.full(groups, parent, np.int64), roots)
            self.alloc.free(parent)
            self.alloc.append(roots, lens[::W.BEAMS] - 1 - W.PREFIX_TOKENS, want_slots=False)
            self.alloc.fork_many(np.repeat(roots, W.BEAMS), self.seqs)
            self.alloc.free_many(roots)
            self.next_id = int(self.seqs[-1]) + 1
            self.beam_rng = np.random.default_rng(shape.seed + 100)
            self.group_base = (np.arange(groups) * W.BEAMS)[:, None]
        elif name == "prefix_shared" and self.duplicate_prefix:
            # the control: every sequence allocates its own prefix blocks (filled below with
            # copies of one sequence's prefix)
            for s in self.seqs:
                self.alloc.add_seq(int(s))
            self.alloc.append(self.seqs, lens - 1, want_slots=False)
        elif name == "prefix_shared":
            prefix = W.PREFIX_TOKENS
            parent = 10_000_000
            self.alloc.add_seq(parent)
            self.alloc.append([parent], [prefix], want_slots=False)
            for s in self.seqs:
                self.alloc.fork(parent, int(s))
            self.alloc.free(parent)  # the children keep the prefix blocks alive
            self.alloc.append(self.seqs, lens - 1 - prefix, want_slots=False)
        else:
            for s in self.seqs:
                self.alloc.add_seq(int(s))
            self.alloc.append(self.seqs, lens - 1, want_slots=False)
        self.max_ctx = int(lens.max()) + total_steps
        self.max_blocks = -(-self.max_ctx // 16)
        dev = "cuda"
        self.k_cache, self.v_cache = pkv.alloc_caches(nb, self.Hkv, self.hd, self.dt, dev)
        self.k_cache.view(-1).copy_(W.device_normal((self.k_cache.numel(),), shape.dtype, 7001))
        self.v_cache.view(-1).copy_(W.device_normal((self.v_cache.numel(),), shape.dtype, 7002))
        if self.duplicate_prefix:  # each sequence's prefix blocks hold sequence 0's prefix
            tab, _ = self.alloc.tables(self.seqs, W.blocks_for(int(lens.max())))
            pb = W.PREFIX_TOKENS // 16
            src = torch.from_numpy(np.repeat(tab[:1, :pb], self.B - 1, axis=0).reshape(-1)
                                   .astype(np.int64)).to(dev)
            dst = torch.from_numpy(tab[1:, :pb].reshape(-1).astype(np.int64)).to(dev)
            self.k_cache[dst] = self.k_cache[src]
            self.v_cache[dst] = self.v_cache[src]
        self.q = W.device_normal((self.B, self.Hq, self.hd), shape.dtype, 7003)
        self.k_new = W.device_normal((self.B, self.Hkv, self.hd), shape.dtype, 7004)
        self.v_new = W.device_normal((self.B, self.Hkv, self.hd), shape.dtype, 7005)
        self.out = torch.empty_like(self.q)
        # Two sets of step buffers, each one packed int32 array [lens | slots | copy-on-write
        # sources | copy-on-write targets | tables | shared-prefix plan], in pinned host memory
        # and on the device: the host prepares step k+1 and its copy runs on a copy stream
        # while step k's kernels run on the compute stream.
        self.plan0 = 4 * self.B + self.B * self.max_blocks
        cap = int(pkv.lib.pkv_decode_plan_max_ints(self.B, self.max_blocks)) if self.planned else 0
        n_int = self.plan0 + cap
        self.plan_len = [0, 0]
        self.pin = [torch.empty(n_int, dtype=torch.int32, pin_memory=True) for _ in range(2)]
        self.dev = [torch.empty(n_int, dtype=torch.int32, device=dev) for _ in range(2)]
        self.host_views = [self._views(t.numpy()) for t in self.pin]
        self.dev_views = [self._views(t) for t in self.dev]
        self.copy_stream = torch.cuda.Stream()
        self.copied = [torch.cuda.Event() for _ in range(2)]
        # a step's completion (its device buffer set may then be refilled): fence-less events,
        # like the timing ones, so the marker between steps does no cache writeback
        self.done = [TimingEvent() for _ in range(2)]
        self.step_no = 0
        # Both sets start from a full export of the allocator's tables; after that each step
        # only adds the blocks it opened (tables only grow in a decode loop without forks).
        for lens_h, _, tables_h in self.host_views:  # shared blocks marked for cached loads
            self.alloc.tables(self.seqs, self.max_blocks, tables_out=tables_h, lens_out=lens_h,
                              mark_shared=True)
        self.lens = self.host_views[0][0].copy()  # lengths before the next step's token
        self.pending = [[], []]  # table entries set s has not received yet
        self.rows = np.arange(self.B)
        self.ones = np.ones(self.B, np.int32)
        self.kernel = pkv.pkv_decode_kernel(self.Hq, self.Hkv, self.dt)
        self.W = pkv.pkv_decode_num_workers(self.Hq, self.Hkv, self.hd, self.dt)
        nbytes = pkv.pkv_decode_stream_workspace_bytes(self.B, self.Hq, self.Hkv, self.hd,
                                                       self.dt, self.W)
        self.ws_dev = dev
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        for e in self.done:
            e.record()
        self.scale = 1.0 / math.sqrt(self.hd)
        self.skips = []  # per timed step: each sequence's shared blocks (planned runs)
        # the library's step engine: one call per step (re-selection for beams, append, table
        # and plan export + upload, copy-on-write copies, the decode kernels)
        self.engine = None
        if engine:
            self.engine = pkv.Engine(self.alloc, self.k_cache, self.v_cache, num_q_heads=self.Hq,
                                     num_kv_heads=self.Hkv, head_dim=self.hd, max_batch=self.B,
                                     max_context_len=self.max_ctx, plan=self.planned,
                                     shared_launch=shared_launch)
            self.engine.adopt(self.seqs)

    def launches(self, plan, pkv):
        """Launches (1 or 2) of the shared and stream passes the library's automatic choice
        gives this plan."""
        return pkv.pkv_decode_planned_launches(plan, batch=self.B, num_q_heads=self.Hq,
                                               num_kv_heads=self.Hkv, max_blocks=self.max_blocks,
                                               dtype=self.dt, num_workers=self.W)

    def planned_skip(self):
        """Each sequence's blocks covered by the shared pass this step (zeros unplanned)."""
        return self.step_skip if self.planned else np.zeros(self.B, np.int32)

    def build_plan(self, s, pkv):
        """Shared-prefix plan of buffer set s's tables and lengths, into its pinned region;
        grows the workspace when the plan needs more. Returns the number of ints."""
        lens_h, _, tables_h = self.host_views[s]
        region = self.pin[s].numpy()[self.plan0:]
        plan = pkv.pkv_decode_plan(tables_h, lens_h, num_q_heads=self.Hq, num_kv_heads=self.Hkv,
                                   num_blocks=self.NB, max_context_len=self.max_ctx,
                                   dtype=self.dt, out=region)
        assert plan.base is not None and np.shares_memory(plan, region)
        need = pkv.pkv_decode_planned_workspace_bytes(self.B, self.Hq, self.Hkv, self.hd,
                                                      self.dt, self.W, plan)
        if need > self.workspace.numel():
            self.workspace = self.torch.empty(need, dtype=self.workspace.dtype,
                                              device=self.ws_dev)
        self.plan_len[s] = len(plan)
        self.step_skip = plan[16:16 + self.B].copy()
        return len(plan)

    def _views(self, flat):
        B, mb = self.B, self.max_blocks
        return flat[:B], flat[B:2 * B], flat[4 * B:4 * B + B * mb].reshape(B, mb)

    def cow_views(self, s):
        """(host, device) views [2, B] of buffer set s's copy-on-write pairs."""
        B = self.B
        return self.pin[s].numpy()[2 * B:4 * B].reshape(2, B), self.dev[s][2 * B:4 * B].view(2, B)

    def kv_bytes(self, lens):
        return int(lens.astype(np.int64).sum()) * 2 * self.Hkv * self.hd * self.eb

    def unique_kv_bytes(self, lens, tables, upto=None):
        """K+V bytes of the distinct cache slots the step reads (shared blocks counted once);
        with upto, only each sequence's first upto[i] blocks."""
        j = np.arange(tables.shape[1])[None, :]
        valid = np.clip(lens[:, None].astype(np.int64) - 16 * j, 0, 16)
        if upto is not None:
            valid = np.where(j < np.asarray(upto)[:, None], valid, 0)
        best = np.zeros(self.NB, np.int64)
        m = valid > 0
        np.maximum.at(best, tables[m], valid[m])
        return int(best.sum()) * 2 * self.Hkv * self.hd * self.eb

    def qo_bytes(self):
        """q read and out written, plus the newest token's K/V read from k_new/v_new and
        stored into its slot (the stream pass does the step's cache write)."""
        return 2 * self.B * self.Hq * self.hd * self.eb + 4 * self.B * self.Hkv * self.hd * self.eb


def beam_reselect(wl, s):
    """Beam-search host part of a step: every group's next beams fork from seeded parents
    among its current beams, the old beams are freed, each new beam appends one token, and
    buffer set s receives the full table export and the copy-on-write pairs. Returns the
    number of pairs."""
    lens_h, _, tables_h = wl.host_views[s]
    cow_h, _ = wl.cow_views(s)
    pick = wl.gen.beam_parents(wl.beam_rng, wl.group_base.shape[0], wl.gen.BEAMS)
    parents = wl.seqs[(wl.group_base + pick).reshape(-1)]
    children = np.arange(wl.next_id, wl.next_id + wl.B, dtype=np.int64)
    wl.next_id += wl.B
    wl.alloc.fork_many(parents, children)
    wl.alloc.free_many(wl.seqs)
    wl.seqs = children
    _, cows = wl.alloc.append(wl.seqs, wl.ones, want_slots=False)
    wl.alloc.tables(wl.seqs, wl.max_blocks, tables_out=tables_h, lens_out=lens_h,
                    mark_shared=True)
    n = len(cows)
    cow_h[:, :n] = cows.T
    wl.lens = lens_h.copy()
    return n


def run_step(wl, torch, pkv, events=None):
    """One decode step (see the module docstring). Returns the context lengths it used and,
    for beam search, the step's tables."""
    if wl.engine is not None:
        return run_engine_step(wl, events)
    s = wl.step_no % 2
    wl.step_no += 1
    wl.done[s].synchronize()  # the step that last used buffer set s has finished
    if wl.beam:
        return run_beam_step(wl, torch, pkv, s, events)
    lens_h, slots_h, tables_h = wl.host_views[s]
    wl.alloc.append(wl.seqs, wl.ones, slots_out=slots_h)  # 1. allocate on demand
    opened = wl.lens % 16 == 0  # the new token is the first of a fresh block
    update = (wl.rows[opened], wl.lens[opened] // 16, slots_h[opened] // 16)
    wl.lens += 1
    wl.pending[0].append(update)
    wl.pending[1].append(update)
    for r, c, b in wl.pending[s]:  # 2. this set's table rows catch up, lengths refreshed
        tables_h[r, c] = b
    wl.pending[s].clear()
    lens_h[:] = wl.lens
    with torch.cuda.stream(wl.copy_stream):  # 2. tables, lengths, slots (and plan) to the device
        if wl.planned:
            n = wl.plan0 + wl.build_plan(s, pkv)
            wl.dev[s][:n].copy_(wl.pin[s][:n], non_blocking=True)
        else:
            wl.dev[s].copy_(wl.pin[s], non_blocking=True)
        wl.copied[s].record(wl.copy_stream)
    # The host waits for the small upload (the device is still on the previous step), so the
    # compute stream needs no cross-stream wait: a device-side wait measured 5 us per step.
    wl.copied[s].synchronize()
    attend(wl, pkv, s, events)  # no copy-on-write in a decode loop without forks
    return lens_h.copy(), (tables_h.copy() if wl.planned else None), wl.planned_skip()


def marked_prefix(tables, lens):
    """Each row's leading blocks whose entries carry the shared mark (within its length): the
    blocks a shared-prefix plan's runs cover when every holder of a shared block is in the
    batch, as in these workloads."""
    nblk = -(-lens.astype(np.int64) // 16)
    j = np.arange(tables.shape[1])[None, :]
    mark = ((tables & 0x40000000) != 0) & (tables >= 0) & (j < nblk[:, None])
    return np.where(mark.all(axis=1), nblk, np.argmin(mark, axis=1)).astype(np.int32)


def run_engine_step(wl, events=None):
    """One decode step as one engine call (pkv_engine_beam_step): for beam search the
    re-selection (seeded parents, fresh child ids), then one token appended per sequence,
    the tables (and the plan) exported and uploaded, the copy-on-write copies and the decode
    kernels launched. Events as attend()'s: [0] before the copies, [1] before the shared
    pass, [2] before the stream pass, [3] before the merge, [4] after it; and [5] before the
    engine's staging upload (which [0] follows)."""
    wl.step_no += 1
    parents = children = None
    if wl.beam:
        pick = wl.gen.beam_parents(wl.beam_rng, wl.group_base.shape[0], wl.gen.BEAMS)
        parents = (wl.group_base + pick).reshape(-1).astype(np.int32)
        children = np.arange(wl.next_id, wl.next_id + wl.B, dtype=np.int64)
        wl.next_id += wl.B
        wl.seqs = children
    # beam steps stage and copy in one launch: no event between the two ([0] is not recorded)
    ev = None if events is None else [events[5], None if wl.beam else events[0], None, events[1],
                                      None, events[2], events[3], events[4]]
    info = wl.engine.beam_step(wl.q, wl.k_new, wl.v_new, wl.out, scale=wl.scale,
                               parents=parents, children=children, events=ev)
    if wl.beam:
        wl.cows.append(int(info[5]))
        wl.cows_all.append(int(info[5]))
    if wl.planned or wl.beam:  # the step's tables (a planned step's shared blocks are found
        # after the timed loop, marked_prefix)
        wl.lens, wl.last_tables = wl.engine.last_tables()
        return wl.lens, wl.last_tables, None if wl.planned else wl.planned_skip()
    # a decode loop's tables only gain entries: the final ones serve every step
    wl.lens = wl.engine.last_lens()
    return wl.lens, None, wl.planned_skip()


def run_beam_step(wl, torch, pkv, s, events):
    ncow = beam_reselect(wl, s)
    wl.cows.append(ncow)
    wl.cows_all.append(ncow)
    n = wl.plan0 + (wl.build_plan(s, pkv) if wl.planned else 0)
    with torch.cuda.stream(wl.copy_stream):  # tables, lengths, pairs (and plan) to the device
        wl.dev[s][:n].copy_(wl.pin[s][:n], non_blocking=True)
        wl.copied[s].record(wl.copy_stream)
    wl.copied[s].synchronize()  # as in run_step: waited on the host, not on the device
    if events is not None:
        events[0].record()
    if ncow:  # copy-on-write: the shared blocks appenders moved off, copied to their new blocks
        _, cow_d = wl.cow_views(s)
        pkv.pkv_copy_blocks(wl.k_cache, wl.v_cache, cow_d[0, :ncow], cow_d[1, :ncow],
                            num_kv_heads=wl.Hkv, head_dim=wl.hd)
    attend(wl, pkv, s, events)
    return wl.lens.copy(), wl.host_views[s][2].copy(), wl.planned_skip()


def attend(wl, pkv, s, events):
    """The step's kernels on buffer set s (tables, lengths and plan on the device): the
    stream pass (with the newest tokens) and the merge (which also stores them), after the
    shared pass when the batch is planned. Events: [1] before the shared pass, [2] before the
    stream pass, [3] before the merge, [4] after it."""
    lens_d, _, tables_d = wl.dev_views[s]

    def mark(k):
        if events is not None:
            events[k].record()
    if events is not None and wl.beam:
        events[1].record()  # [0]: before the copy-on-write copies
    elif events is not None:
        events[0].record()  # [0] == [1]: no copy-on-write here
    if wl.planned:
        plan = wl.pin[s].numpy()[wl.plan0:wl.plan0 + wl.plan_len[s]]
        plan_d = wl.dev[s][wl.plan0:wl.plan0 + wl.plan_len[s]]
        form = wl.shared_launch
        if form == "auto" and events is not None:  # the events between the kernels it runs
            form = "one" if wl.launches(plan, pkv) == 1 else "two"
        pkv.pkv_decode_planned(wl.q, wl.k_cache, wl.v_cache, tables_d, lens_d, plan, plan_d,
                               num_kv_heads=wl.Hkv, scale=wl.scale, max_context_len=wl.max_ctx,
                               num_workers=wl.W, workspace=wl.workspace, k_new=wl.k_new,
                               v_new=wl.v_new, out=wl.out,
                               events=None if events is None else events[2:5],
                               shared_launch=form)
    else:  # [2] == [1]: no shared pass
        # 3 + 4a. cache write of the newest tokens fused into the attention stream pass
        pkv.pkv_decode_append_stream(wl.q, wl.k_new, wl.v_new, wl.k_cache, wl.v_cache, tables_d,
                                     lens_d, num_kv_heads=wl.Hkv, scale=wl.scale,
                                     max_context_len=wl.max_ctx, num_workers=wl.W,
                                     workspace=wl.workspace, out=wl.out)
        mark(3)
        # 4b. merge of the cut segments, plus the stores of the new tokens into their slots
        pkv.pkv_decode_append_merge(wl.out, wl.k_new, wl.v_new, wl.k_cache, wl.v_cache,
                                    tables_d, lens_d, wl.workspace, num_kv_heads=wl.Hkv,
                                    max_context_len=wl.max_ctx, num_workers=wl.W)
        mark(4)
    wl.done[s].record()
    wl.last_set = s


def bandwidth_probe(torch, pkv, waves, reps=10):
    """Attainable read bandwidth on this part (pkv_probe_read) with `waves` waves: 2 GiB of 4 KiB
    tiles read with the stream pass's loads and none of its arithmetic, over consecutive tiles
    (each wave a contiguous range) and over a random permutation (the decode path's gather
    pattern); median of `reps` launches timed with HIP events, after the timed region."""
    nbytes = 2 << 30
    n = nbytes // 4096
    base = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty(waves * 64, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(99)
    res = {"bytes_per_launch": nbytes, "waves": waves}
    for name, ids in (("sequential_4k_tiles", np.arange(n)), ("random_4k_tiles", rng.permutation(n))):
        d_ids = torch.from_numpy(ids.astype(np.int32)).cuda()
        for _ in range(2):
            pkv.pkv_probe_read(base, d_ids, num_workers=waves, sink=sink)
        ms = []
        for _ in range(reps):
            e0, e1 = TimingEvent(), TimingEvent()
            e0.record()
            pkv.pkv_probe_read(base, d_ids, num_workers=waves, sink=sink)
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        res[f"{name}_gbs"] = round(nbytes / (float(np.median(ms)) / 1e3) / 1e9, 1)
    del base, sink
    torch.cuda.empty_cache()
    return res


def cpu_baseline(wl, torch, W, seconds):
    """The oracle (float64 NumPy) on the last step's sequences, in a seeded order: first on one
    thread, then on a pool of one thread per available core (at most 16), each for about half of
    ``seconds``."""
    if wl.engine is not None:
        lens, tables = wl.lens, wl.last_tables
    else:
        lens, tables = wl.host_views[wl.last_set][0], wl.host_views[wl.last_set][2]
    return oracle_baseline(torch, W, seconds, lens, tables, wl.k_cache, wl.v_cache, wl.q,
                           wl.Hkv, wl.hd, wl.shape.dtype, wl.scale)


def oracle_baseline(torch, W, seconds, lens, tables, k_cache, v_cache, q_all, Hkv, hd, dtype,
                    scale):
    import concurrent.futures
    import threading

    from threadpoolctl import threadpool_limits

    from oracle import attention as OA
    B = len(lens)
    eb = 4 if dtype == "f32" else 2
    order = np.random.default_rng(12345).permutation(B)
    lens = np.array(lens, copy=True)
    tables = np.array(tables, copy=True)
    tables = np.where(tables >= 0, tables & ~0x40000000, tables)  # drop the shared-block mark
    inputs = {}
    for i in order:  # exact host copies of each sequence's blocks (untimed)
        n = int(lens[i])
        nbk = -(-n // 16)
        ids = torch.from_numpy(tables[i, :nbk].astype(np.int64)).cuda()
        inputs[int(i)] = (n, nbk,
                          W.to_storage_numpy(k_cache.index_select(0, ids), dtype).reshape(-1),
                          W.to_storage_numpy(v_cache.index_select(0, ids), dtype).reshape(-1),
                          W.to_storage_numpy(q_all[i:i + 1], dtype))

    def attend(i):
        n, nbk, kc, vc, q = inputs[i]
        OA.decode_attention(q, kc, vc, np.arange(nbk, dtype=np.int32)[None], np.int32([n]),
                            scale=scale, hkv=Hkv, hd=hd, bs=16, dtype=dtype)
        return n * 2 * Hkv * hd * eb

    def tasks():  # the seeded order, pass after pass
        while True:
            for i in order:
                yield int(i)

    budget = seconds / 2
    # one thread
    done1, kv1, t0 = 0, 0, time.perf_counter()
    with threadpool_limits(limits=1):
        for i in tasks():
            kv1 += attend(i)
            done1 += 1
            if time.perf_counter() - t0 >= budget:
                break
    wall1 = time.perf_counter() - t0
    # a pool of one thread per available core; each worker takes tasks until the budget is spent
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    lock = threading.Lock()
    it = tasks()
    stats = {"done": 0, "kv": 0}
    t0 = time.perf_counter()

    def worker():
        while time.perf_counter() - t0 < budget:
            with lock:
                i = next(it)
            kv = attend(i)
            with lock:
                stats["done"] += 1
                stats["kv"] += kv

    with threadpool_limits(limits=1):
        with concurrent.futures.ThreadPoolExecutor(max_workers=cores) as ex:
            for f in [ex.submit(worker) for _ in range(cores)]:
                f.result()
    wall = time.perf_counter() - t0
    pool = stats["kv"] / wall / 1e9
    single = kv1 / wall1 / 1e9
    pool_sample = (f"{stats['done']} sequence-attentions, {stats['kv'] / 1e6:.1f} MB of K/V, "
                   f"{wall:.1f} s wall on {cores} threads (one per available core, BLAS on one "
                   f"thread each)")
    single_sample = f"{done1} sequence-attentions, {kv1 / 1e6:.1f} MB of K/V, {wall1:.1f} s on one thread"
    # the better of the two configurations is the baseline; cores = the threads it used
    use_pool = pool > single
    return {"value": round(max(pool, single), 4), "unit": "GB/s", "cores": cores if use_pool else 1,
            "kind": "oracle",
            "sample": f"the step's {B} sequences in a seeded order, host copies of their blocks "
                      f"not timed; " + (pool_sample if use_pool else single_sample) +
                      f" (the better of one thread and a {cores}-thread pool)",
            "tokens_per_s_per_layer": round(stats["done"] / wall if use_pool else done1 / wall1, 3),
            "single_thread_value": round(single, 4), "single_thread_sample": single_sample,
            "pool_value": round(pool, 4), "pool_cores": cores, "pool_sample": pool_sample}


BATCHING = {
    "continuous_batching": dict(shape=("f16", 32, 32, 128), max_batch=64, max_ctx=2048,
                                pool_blocks=4096, prompt=(64, 1024), new=(16, 256), rate=0.5,
                                requests=4000, seed=7, settle_steps=300, system=0),
    "prefix_cache": dict(shape=("bf16", 28, 4, 128), max_batch=128, max_ctx=2560,
                         pool_blocks=24576, prompt=(16, 256), new=(16, 256), rate=1.0,
                         requests=4000, seed=8, settle_steps=300, system=2000),
}


def batching_main(args, torch, pkv, W):
    """The continuous-batching workloads: one engine call per step (retire, admit + prompt
    write, decode), timed over K steps after W warm-up steps."""
    from paged_kv_cache_459_amd.batching import ContinuousBatch
    cfg = BATCHING[args.workload]
    dtype, Hq, Hkv, hd = cfg["shape"]
    dt = W.torch_dtype(dtype)
    rng = np.random.default_rng(cfg["seed"])
    reqs = W.request_stream(rng, cfg["requests"], prompt=cfg["prompt"], new=cfg["new"],
                            rate=cfg["rate"])
    cache_on = cfg["system"] > 0
    system = rng.integers(0, 32000, size=cfg["system"]).astype(np.int32)
    nb = cfg["pool_blocks"]
    k_cache, v_cache = pkv.alloc_caches(nb, Hkv, hd, dt)
    k_cache.view(-1).copy_(W.device_normal((k_cache.numel(),), dtype, 7101))
    v_cache.view(-1).copy_(W.device_normal((v_cache.numel(),), dtype, 7102))
    loop = ContinuousBatch(k_cache, v_cache, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=hd,
                           max_batch=cfg["max_batch"], max_context_len=cfg["max_ctx"],
                           free_order=rng.permutation(nb).astype(np.int32),
                           prefix_cache=cache_on)
    for i, (rid, p, m, a) in enumerate(reqs):  # the first max_batch requests are a backlog
        arrival = 0 if i < cfg["max_batch"] else a + 1
        if cache_on:
            ids = np.concatenate([system, rng.integers(0, 32000, size=p).astype(np.int32)])
            loop.submit(rid, len(ids), m, arrival, token_ids=ids)
        else:
            loop.submit(rid, p, m, arrival)
    B = cfg["max_batch"]
    q = W.device_normal((B, Hq, hd), dtype, 7103)
    k_new = W.device_normal((B, Hkv, hd), dtype, 7104)
    v_new = W.device_normal((B, Hkv, hd), dtype, 7105)
    max_prompt = (cfg["prompt"][1] + cfg["system"]) * cfg["max_batch"]
    k_prompt = W.device_normal((max_prompt, Hkv, hd), dtype, 7106)
    v_prompt = W.device_normal((max_prompt, Hkv, hd), dtype, 7107)
    out = torch.empty_like(q)
    scale = 1.0 / math.sqrt(hd)
    eb = 2
    q_prompt = (W.device_normal((max_prompt, Hq, hd), dtype, 7108) if args.with_prefill
                else None)
    pf_out = torch.empty_like(q_prompt) if args.with_prefill else None

    ids_rng = np.random.default_rng(cfg["seed"] + 1)
    q_pf = q_prompt if args.with_prefill else None

    def step(ev=None, stats=None):
        """One engine call: retire, admit + prompt write (+ prefill), decode. Events (8, when
        given): before the staging upload, after it, after the prompt write, after the
        copy-on-write copies, after the prefill, after the shared pass, after the stream pass,
        after the merge."""
        new_ids = ids_rng.integers(0, 32000, size=B).astype(np.int32) if cache_on else None
        info = loop.step(q, k_new, v_new, out, scale=scale, k_prompt=k_prompt,
                         v_prompt=v_prompt, q_prompt=q_pf, prefill_out=pf_out, new_ids=new_ids,
                         events=ev)
        if stats is not None:
            n, T = int(info[0]), int(info[1])
            last = loop.last()
            pf_flops = 0.0
            if args.with_prefill:
                for _, p, c in last["admitted"]:
                    pf_flops += 4.0 * hd * Hq * (p * (p + 1) / 2 - c * (c + 1) / 2)
            lens = last["lens"]
            u = loop.usage() if ev is not None else None  # sampled: it walks every block
            stats.append(dict(B=n, retired=int(info[2]), admitted=int(info[3]), T=T,
                              pf_flops=pf_flops, planned=int(info[4]) > 0,
                              prompt=sum(a[1] for a in last["admitted"]),
                              kv=int(lens.astype(np.int64).sum()) * 2 * Hkv * hd * eb,
                              lens=lens, tables=last["tables"], usage=u))

    # events created and recorded once before the warm-up (see main)
    every = 1 if args.flush else max(1, args.event_every)
    timed = [k for k in range(args.steps) if k % every == 0]
    evs = {k: [TimingEvent() for _ in range(8)] for k in timed}
    prime(torch, [e for v in evs.values() for e in v])
    scratch = flush_buffer(torch) if args.flush else None
    for _ in range(cfg["settle_steps"] + args.warmup):
        step()
    step([TimingEvent() for _ in range(8)])  # the event path warm before the timed region
    stats = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        if scratch is not None:  # before the step's events: not part of the kernels' times
            flush(scratch)
        step(evs.get(k), stats)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    staging_ms = [evs[k][0].elapsed_time(evs[k][1]) for k in timed]
    write_ms = [evs[k][1].elapsed_time(evs[k][2]) for k in timed]
    prefill_ms = ([evs[k][3].elapsed_time(evs[k][4]) for k in timed] if args.with_prefill
                  else None)
    shared_ms = [evs[k][4].elapsed_time(evs[k][5]) for k in timed]
    part_ms = [evs[k][5].elapsed_time(evs[k][6]) for k in timed]
    merge_ms = [evs[k][6].elapsed_time(evs[k][7]) for k in timed]
    step_kernel_ms = [evs[k][0].elapsed_time(evs[k][7]) for k in timed]

    def unique(lens, tables):  # K+V bytes of the distinct cache slots read
        t = np.where(tables >= 0, tables & ~pkv.BLOCK_SHARED, tables)
        j = np.arange(t.shape[1])[None, :]
        valid = np.clip(lens[:, None].astype(np.int64) - 16 * j, 0, 16)
        best = np.zeros(nb, np.int64)
        m = (valid > 0) & (t >= 0)
        np.maximum.at(best, t[m], valid[m])
        return int(best.sum()) * 2 * Hkv * hd * eb
    kv_logical = [st["kv"] for st in stats]
    kv = [unique(st["lens"], st["tables"]) for st in stats]
    # with a plan the stream pass reads only the unshared blocks: the blocks whose table entry
    # is not marked shared (the plan's runs are exactly the shared prefixes of the tables)
    kv_private = [unique(st["lens"], np.where(st["tables"] & 0x40000000, -1, st["tables"]))
                  if st["planned"] else k for st, k in zip(stats, kv)]
    qo = [2 * st["B"] * Hq * hd * eb + 4 * st["B"] * Hkv * hd * eb for st in stats]
    algo = [kv_private[k] + qo[k] for k in timed]
    attn_ms = [a + b + c for a, b, c in zip(shared_ms, part_ms, merge_ms)]
    if args.flush:  # the steps are separated by the flushes: the step's kernels' own times
        ms_per_step = float(np.mean(step_kernel_ms))
        wall_eff = sum(step_kernel_ms) / 1e3
    else:
        ms_per_step = wall / args.steps * 1e3
        wall_eff = wall
    tokens = sum(st["B"] for st in stats)
    kv_t = [kv[k] for k in timed]
    qo_t = [qo[k] for k in timed]
    written_t = sum(stats[k]["T"] for k in timed) * 2 * Hkv * hd * eb
    if args.copy_calibration:  # a plain copy of known size, for the counter runs
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    sampled = [st for st in stats if st["usage"] is not None]
    util_paged = [st["usage"]["utilisation"] for st in sampled]
    util_contig = [st["usage"]["logical_tokens"] / (st["usage"]["sequences"] * cfg["max_ctx"])
                   for st in sampled]
    sharing = [st["usage"]["logical_tokens"] / st["usage"]["slots_filled"] for st in sampled]
    achieved = sum(algo) / (sum(part_ms) / 1e3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(sum(kv) / wall_eff / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded request stream, seeded N(0,1) values and block placement)",
        "timing": {
            "flushed": bool(args.flush),
            "steps_with_kernel_events": len(timed),
            "note": ("a 1 GiB scratch read before every timed step; value and ms_per_step are "
                     "the step's kernels' event times" if args.flush else
                     "back-to-back steps; value and ms_per_step are wall-clock over every step, "
                     "kernel times from the events of every n-th step"),
            "kernel_ms": {name: ms_stats(v) for name, v in
                          (("staging_upload", staging_ms), ("prompt_write", write_ms),
                           ("shared", shared_ms), ("stream", part_ms), ("merge", merge_ms),
                           ("attention", attn_ms), ("step", step_kernel_ms))},
        },
        "config": {"workload": args.workload, "description": DESC[args.workload],
                   "with_prefill": bool(args.with_prefill),
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": hd, "block_size": 16,
                   "pool_blocks": nb, "max_batch": cfg["max_batch"],
                   "max_context_len": cfg["max_ctx"], "stream_workers": loop.W,
                   "attn_kernel": ["", "vector", "matrix-core"][loop.kernel]},
        "tokens_per_s_per_layer": round(tokens / wall_eff, 1),
        "attn_stream_ms": round(float(np.mean(part_ms)), 4),
        "attn_merge_ms": round(float(np.mean(merge_ms)), 4),
        "attn_shared_ms": round(float(np.mean(shared_ms)), 4),
        "attention_unique_gbs": round((sum(kv_t) + sum(qo_t)) / (sum(attn_ms) / 1e3) / 1e9, 2),
        "step": {
            "note": "one pkv_engine_step call per step (retire, admit, prompt write, decode); "
                    "kernel_ms is the device time from before the step's first kernel (the "
                    "staging upload) to the end of its merge, on the steps that record events",
            "calls_per_step": 1,
            "kernel_ms": ms_stats(step_kernel_ms),
            "staging_upload_ms": ms_stats(staging_ms),
            "wall_over_kernel": round(ms_per_step / float(np.mean(step_kernel_ms)), 4),
        },
        "batching": {
            "mean_running": round(tokens / args.steps, 2),
            "prefix_cache": cache_on,
            "planned_steps": sum(st["planned"] for st in stats),
            "prompt_tokens_admitted_per_step": round(sum(st["prompt"] for st in stats)
                                                     / args.steps, 1),
            "admitted_per_step": round(sum(st["admitted"] for st in stats) / args.steps, 3),
            "retired_per_step": round(sum(st["retired"] for st in stats) / args.steps, 3),
            "prompt_tokens_written_per_step": round(sum(st["T"] for st in stats) / args.steps, 1),
            "prompt_write_ms_per_step": round(float(np.mean(write_ms)), 4),
            "prompt_write_gbs": (round(written_t / (sum(write_ms) / 1e3) / 1e9, 2)
                                 if written_t else None),
            "mean_context_len": round(float(np.mean(np.concatenate([st["lens"] for st in stats]))),
                                      1),
            "kv_utilisation_paged": round(float(np.mean(util_paged)), 4),
            "kv_utilisation_contiguous_2048": round(float(np.mean(util_contig)), 4),
            "requests_the_pool_holds_contiguous": nb * 16 // cfg["max_ctx"],
            "logical_tokens_per_filled_slot": round(float(np.mean(sharing)), 3),
            "kv_bytes_per_step": {"unique": int(np.mean(kv)), "logical": int(np.mean(kv_logical))},
        },
        "prefill": None if prefill_ms is None else {
            "note": "each step also attends the admitted prompts' tokens causally "
                    "(pkv_prefill_attn); prompt_write_ms_per_step includes it",
            "ms_per_step": round(float(np.mean(prefill_ms)), 4),
            "tflops": (round(sum(stats[k]["pf_flops"] for k in timed) / (sum(prefill_ms) / 1e3)
                             / 1e12, 2) if sum(prefill_ms) > 0 else None),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(args.workload, kernel_source_digest(args.workload)),
            "kernel": f"attention stream pass ({['', 'vector', 'matrix-core'][loop.kernel]} "
                      f"kernel)",
            "algorithmic_bytes_per_launch": int(np.mean(algo)),
        },
    }
    if not args.no_cpu_baseline:
        last = stats[-1]
        res["cpu_baseline"] = oracle_baseline(torch, W, args.cpu_seconds, last["lens"],
                                              last["tables"], k_cache, v_cache, q, Hkv, hd,
                                              dtype, scale)
    print(json.dumps(res), flush=True)


def prefill_main(args, torch, pkv, W):
    """The chunked-prefill workload: one step = pkv_write of the new tokens' K/V, then the
    causal attention of those tokens over their sequences' paged caches."""
    shape = W.SHAPES["prefill"]
    dtype, Hq, Hkv, hd = shape.dtype, shape.Hq, shape.Hkv, shape.hd
    dt = W.torch_dtype(dtype)
    rng = W.rng_for(shape.seed)
    lens, qlens = W.prefill_lengths(rng, shape.B)
    nb = W.pool_blocks(lens)
    tables = W.place_sequences(lens, rng.permutation(nb).astype(np.int32))
    mb = tables.shape[1]
    max_ctx = 16 * mb
    qs = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    T = int(qs[-1])
    k_cache, v_cache = pkv.alloc_caches(nb, Hkv, hd, dt)
    k_cache.view(-1).copy_(W.device_normal((k_cache.numel(),), dtype, 7201))
    v_cache.view(-1).copy_(W.device_normal((v_cache.numel(),), dtype, 7202))
    q = W.device_normal((T, Hq, hd), dtype, 7203)
    k_new = W.device_normal((T, Hkv, hd), dtype, 7204)
    v_new = W.device_normal((T, Hkv, hd), dtype, 7205)
    # the new tokens' slots: row t of sequence s sits at position pos = n_s - q_s + k
    slots = np.empty(T, np.int32)
    vis = np.empty(T, np.int64)
    for s_ in range(shape.B):
        pos = np.arange(lens[s_] - qlens[s_], lens[s_])
        slots[qs[s_]:qs[s_ + 1]] = tables[s_, pos // 16] * 16 + pos % 16
        vis[qs[s_]:qs[s_ + 1]] = pos + 1
    slots_dev = torch.from_numpy(slots).cuda()
    tables_dev = torch.from_numpy(tables).cuda()
    t0 = time.perf_counter()
    for _ in range(5):
        plan = pkv.pkv_prefill_plan(qs, lens, num_q_heads=Hq, num_kv_heads=Hkv, max_blocks=mb,
                                    max_context_len=max_ctx, dtype=dt)
    plan_ms = (time.perf_counter() - t0) / 5 * 1e3
    plan_dev = torch.from_numpy(plan.copy()).cuda()
    ws_bytes = pkv.pkv_prefill_workspace_bytes(Hq, Hkv, hd, plan)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    scale = 1.0 / math.sqrt(hd)
    split_rows = int(plan[16:16 + T].sum())

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        pkv.pkv_write(k_new, v_new, k_cache, v_cache, slots_dev)
        if ev is not None:
            ev[1].record()
        for ps in (1, 2):
            pkv.pkv_prefill_attn(q, k_cache, v_cache, tables_dev, plan, plan_dev,
                                 num_kv_heads=Hkv, scale=scale, max_context_len=max_ctx,
                                 workspace=ws, out=out, passes=ps)
            if ev is not None:
                ev[1 + ps].record()

    evs = [[TimingEvent() for _ in range(4)] for _ in range(args.steps)]
    prime(torch, [e for v in evs for e in v])  # before the warm-up (see main)
    for _ in range(args.warmup):
        step()
    step([TimingEvent() for _ in range(4)])  # the event path warm before the timed region
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    write_ms = [e[0].elapsed_time(e[1]) for e in evs]
    attn_ms = [e[1].elapsed_time(e[2]) for e in evs]
    merge_ms = [e[2].elapsed_time(e[3]) for e in evs]
    eb = 2
    flops = 4.0 * hd * Hq * float(vis.sum())  # q.k and p.v over every visible key, per head
    achieved = flops / (float(np.mean(attn_ms)) / 1e3) / 1e12
    kv_bytes = int(lens.astype(np.int64).sum()) * 2 * Hkv * hd * eb
    qo_bytes = 2 * T * Hq * hd * eb
    if args.copy_calibration:  # a plain copy of known size, for the counter runs
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    ms_per_step = wall / args.steps * 1e3
    res = {
        "metric": PREFILL_METRIC,
        "value": round(T / (ms_per_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded N(0,1) values, seeded lengths and block placement)",
        "config": {"workload": "prefill", "description": DESC["prefill"], "sequences": shape.B,
                   "query_tokens": T, "q_heads": Hq, "kv_heads": Hkv, "head_dim": hd,
                   "block_size": 16, "pool_blocks": nb,
                   "mean_context_len": round(float(lens.mean()), 1),
                   "split_rows": split_rows, "plan_units": int(plan[4])},
        "attn_ms": round(float(np.mean(attn_ms)), 4),
        "merge_ms": round(float(np.mean(merge_ms)), 4),
        "write_ms": round(float(np.mean(write_ms)), 4),
        "plan_host_ms": round(plan_ms, 3),
        "attention_tflops": round(flops / ((sum(attn_ms) + sum(merge_ms)) / args.steps / 1e3)
                                  / 1e12, 2),
        "attention_min_bytes_gbs": round((kv_bytes + qo_bytes) / (float(np.mean(attn_ms)) / 1e3)
                                         / 1e9, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": MFMA_PEAK_TFLOPS[dtype],
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_PEAK_TFLOPS[dtype], 4),
            "traffic": measured_traffic("prefill", kernel_source_digest("prefill")),
            "kernel": "prefill attention pass (attn_prefill_kernel)",
            "algorithmic_flops_per_launch": flops,
        },
    }
    if not args.no_cpu_baseline:
        # the oracle on whole sequences' new tokens, in a seeded order, until the budget is spent
        from threadpoolctl import threadpool_limits

        from oracle import attention as OA
        order = np.random.default_rng(12345).permutation(shape.B)
        spent, rows, fl, seqs = 0.0, 0, 0.0, 0
        with threadpool_limits(limits=1):
            for s_ in order:
                n = int(lens[s_])
                nbk = -(-n // 16)
                ids = torch.from_numpy(tables[s_, :nbk].astype(np.int64)).cuda()
                kc = W.to_storage_numpy(k_cache.index_select(0, ids), dtype).reshape(-1)
                vc = W.to_storage_numpy(v_cache.index_select(0, ids), dtype).reshape(-1)
                a, b = int(qs[s_]), int(qs[s_ + 1])
                # a bounded slice of the sequence's rows: its last new tokens
                take = min(b - a, 64)
                qh = W.to_storage_numpy(q[b - take:b], dtype)
                t1 = time.perf_counter()
                OA.prefill_attention(qh, kc, vc, np.arange(nbk, dtype=np.int32)[None],
                                     np.int32([n]), np.int32([0, take]), scale=scale, hkv=Hkv,
                                     hd=hd, bs=16, dtype=dtype)
                spent += time.perf_counter() - t1
                rows += take
                seqs += 1
                fl += 4.0 * hd * Hq * float(vis[b - take:b].sum())
                if spent >= args.cpu_seconds:
                    break
        res["cpu_baseline"] = {
            "value": round(rows / spent, 2), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"the last 64 new tokens of {seqs} sequence(s) in a seeded order: "
                      f"{rows} query tokens, {spent:.1f} s of oracle time on one thread (host "
                      f"copies of the blocks not timed)",
            "tflops": round(fl / spent / 1e12, 6)}
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world})", file=sys.stderr)
        sys.exit(2)
    import torch

    import paged_kv_cache_459_amd as pkv
    import workloads as W

    torch.cuda.set_device(0)
    pkv.pkv_set_attn_kernel(args.kernel)
    if args.workload in BATCHING:
        batching_main(args, torch, pkv, W)
        return
    if args.workload == "prefill":
        prefill_main(args, torch, pkv, W)
        return
    wl = Workload(args.workload, args.warmup + 1 + args.steps, torch, pkv, W, plan=not args.no_plan,
                  duplicate_prefix=args.duplicate_prefix, shared_launch=args.shared_launch,
                  engine=args.driver == "engine" or (args.driver == "auto" and
                                                     args.workload == "beam_search"))
    torch.cuda.synchronize()

    # per-kernel timing events on every n-th timed step (every step with --flush), created and
    # recorded once before the warm-up: between the warm-up and the timed region the device
    # then idles only for the host's few statements (after an idle millisecond, the first
    # timed step's upload took a millisecond more)
    every = 1 if args.flush else max(1, args.event_every)
    timed = [k for k in range(args.steps) if k % every == 0]
    evs = {k: [TimingEvent() for _ in range(6)] for k in timed}
    prime(torch, [e for v in evs.values() for e in v])
    scratch = flush_buffer(torch) if args.flush else None
    for _ in range(args.warmup):
        run_step(wl, torch, pkv)
    # one more, with timing events: the first record of an event has cost milliseconds of host
    # time in a fresh process, which would otherwise land in the timed region
    run_step(wl, torch, pkv, [TimingEvent() for _ in range(6)])
    per_step = []
    wl.cows.clear()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        if scratch is not None:  # before the step's events: not part of the kernels' times
            flush(scratch)
        per_step.append(run_step(wl, torch, pkv, evs.get(k)))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_step = [(lens, t, marked_prefix(t, lens) if sk is None else sk)
                for lens, t, sk in per_step]

    # events a step does not record stand for the one before them (no copy, no shared pass)
    for e in evs.values():
        if not wl.beam:
            e[1] = e[0]
        if not wl.planned:
            e[2] = e[1]
    # the engine stages a beam step and copies its copy-on-write pairs in one launch: that
    # launch is timed as the copies (the staging inside it), and no separate staging is left
    fused_copy = wl.engine is not None and wl.beam
    if fused_copy:
        copy_ms = [evs[k][5].elapsed_time(evs[k][1]) for k in timed]
    else:
        copy_ms = [evs[k][0].elapsed_time(evs[k][1]) if wl.beam else 0.0 for k in timed]
    staging_ms = ([evs[k][5].elapsed_time(evs[k][0]) for k in timed]
                  if wl.engine is not None and not fused_copy
                  else None)
    shared_ms = [evs[k][1].elapsed_time(evs[k][2]) if wl.planned else 0.0 for k in timed]
    part_ms = [evs[k][2].elapsed_time(evs[k][3]) for k in timed]
    merge_ms = [evs[k][3].elapsed_time(evs[k][4]) for k in timed]
    # The last tables sent must be exactly what the allocator exports (for the decode loop,
    # whose tables only gain entries, this checks every incremental update).
    if wl.engine is not None:
        final_tables = wl.engine.last_tables()[1]
        wl.last_tables = final_tables
    else:
        final_tables = wl.host_views[wl.last_set][2].copy()
    ref_tables, ref_lens = wl.alloc.tables(wl.seqs, wl.max_blocks, mark_shared=True)
    if wl.engine is not None:  # the engine refreshes a row's marks only where it re-reads it
        final_cmp = np.where(final_tables >= 0, final_tables & ~pkv.BLOCK_SHARED, final_tables)
        ref_cmp = np.where(ref_tables >= 0, ref_tables & ~pkv.BLOCK_SHARED, ref_tables)
    else:
        final_cmp, ref_cmp = final_tables, ref_tables
    assert np.array_equal(final_cmp, ref_cmp) and np.array_equal(wl.lens, ref_lens), \
        "block tables sent to the device diverged from the allocator's export"

    def unmarked(t):
        return np.where(t >= 0, t & ~pkv.BLOCK_SHARED, t)
    lens_per_step = [lens for lens, _, _ in per_step]
    kv_logical = [wl.kv_bytes(lens) for lens in lens_per_step]
    kv = [wl.unique_kv_bytes(lens, unmarked(final_tables if t is None else t))
          for lens, t, _ in per_step]
    # with a plan: the unique bytes the shared pass reads (blocks before each skip) and the
    # rest, which the stream pass reads
    kv_shared = [wl.unique_kv_bytes(lens, unmarked(final_tables if t is None else t), upto=sk)
                 for lens, t, sk in per_step]
    kv_private = [a - b for a, b in zip(kv, kv_shared)]
    # planned steps: the shared and stream passes' launches per timed step (the automatic
    # choice from each step's plan, rebuilt here from its tables and lengths). One launch: the
    # roofline kernel reads every unique block; two: the stream pass reads the private ones
    launches = [0] * len(timed)
    if wl.planned:
        for n, k in enumerate(timed):
            lens_k, t_k, _ = per_step[k]
            if wl.shared_launch != "auto":
                launches[n] = 1 if wl.shared_launch == "one" else 2
                continue
            plan_k = pkv.pkv_decode_plan(final_tables if t_k is None else t_k, lens_k,
                                         num_q_heads=wl.Hq, num_kv_heads=wl.Hkv,
                                         num_blocks=wl.NB, max_context_len=wl.max_ctx,
                                         dtype=wl.dt)
            launches[n] = wl.launches(plan_k, pkv)
    one_launch = wl.planned and all(x == 1 for x in launches)
    algo = [(kv[k] if x == 1 else kv_private[k]) + wl.qo_bytes() for k, x in zip(timed, launches)]
    attn_ms = [a + b + c for a, b, c in zip(shared_ms, part_ms, merge_ms)]
    kv_t = [kv[k] for k in timed]
    kv_logical_t = [kv_logical[k] for k in timed]
    kv_shared_t = [kv_shared[k] for k in timed]
    if args.flush:  # the steps are separated by the flushes: the kernels' own times
        step_ms = [a + b for a, b in zip(copy_ms, attn_ms)]
        ms_per_step = float(np.mean(step_ms))
        value = sum(kv_t) / (sum(step_ms) / 1e3) / 1e9
    else:
        ms_per_step = wall / args.steps * 1e3
        value = sum(kv) / wall / 1e9
    achieved = sum(algo) / (sum(part_ms) / 1e3) / 1e9
    digest = kernel_source_digest(args.workload)
    traffic = measured_traffic(args.workload, digest)

    if args.copy_calibration:  # a plain copy of known size, for the counter runs
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.shape.dtype,
        "data": "synthetic (seeded N(0,1) values, seeded lengths and block placement)",
        "config": {
            "workload": args.workload,
            "description": DESC[args.workload],
            "batch": wl.B, "q_heads": wl.Hq, "kv_heads": wl.Hkv, "head_dim": wl.hd,
            "block_size": 16, "pool_blocks": wl.NB, "stream_workers": wl.W,
            "mean_context_len": round(float(np.mean([l.mean() for l in lens_per_step])), 1),
            "attn_kernel": ["", "vector", "matrix-core"][wl.kernel],
            "planned": wl.planned,
            "duplicate_prefix": wl.duplicate_prefix,
            "step_driver": "host loop" if wl.engine is None else "pkv_engine_beam_step",
        },
        "tokens_per_s_per_layer": round(wl.B / (ms_per_step / 1e3), 1),
        "hbm_frac_of_step": round(value / HBM_PEAK_GBS, 4),
        "attn_stream_ms": round(float(np.mean(part_ms)), 4),
        "attn_merge_ms": round(float(np.mean(merge_ms)), 4),
        "attn_kv_gbs": round(sum(kv_t) / sum(attn_ms) * 1e3 / 1e9, 2),
        "kv_bytes_per_step": {"unique": int(np.mean(kv)), "logical": int(np.mean(kv_logical))},
        "attn_logical_kv_gbs": round(sum(kv_logical_t) / sum(attn_ms) * 1e3 / 1e9, 2),
        "timing": {
            "flushed": bool(args.flush),
            "steps_with_kernel_events": len(timed),
            "note": ("a 1 GiB scratch read before every timed step; value and ms_per_step are "
                     "the step's kernels' event times" if args.flush else
                     "back-to-back steps; value and ms_per_step are wall-clock over every step, "
                     "kernel times from the events of every n-th step"),
            "kernel_ms": {name: ms_stats(v) for name, v in
                          (("shared_and_stream" if one_launch else "stream", part_ms),
                           ("merge", merge_ms), ("attention", attn_ms))
                          + ((("shared", shared_ms),) if wl.planned and not one_launch else ())
                          + ((("staging_and_cow_copy" if fused_copy else "cow_copy", copy_ms),)
                             if wl.beam else ())
                          + ((("staging_upload", staging_ms),) if staging_ms else ())
                          + ((("step", [a + b + c for a, b, c in
                                        zip(staging_ms, copy_ms, attn_ms)]),)
                             if staging_ms else ())
                          + ((("step", [a + b for a, b in zip(copy_ms, attn_ms)]),)
                             if fused_copy else ())},
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": ("shared pass + stream pass, one launch (attn_fused_kernel)" if one_launch
                       else f"attention stream pass ({['', 'vector', 'matrix-core'][wl.kernel]} "
                            "kernel)"),
            "algorithmic_bytes_per_launch": int(np.mean(algo)),
        },
    }
    if wl.planned:
        sh = sum(kv_shared_t)
        res["shared_prefix_plan"] = {
            "shared_launch": wl.shared_launch,
            "launches_per_step": {"one": launches.count(1), "two": launches.count(2)},
            "shared_pass_ms": None if one_launch else round(float(np.mean(shared_ms)), 4),
            "shared_unique_bytes_per_step": int(np.mean(kv_shared)),
            "private_unique_bytes_per_step": int(np.mean(kv_private)),
            "shared_pass_gbs": (round(sh / (sum(shared_ms) / 1e3) / 1e9, 2)
                                if sh and not one_launch else None),
            "attention_ms": round(float(np.mean(attn_ms)), 4),
            "attention_unique_gbs": round((sum(kv_t) + len(timed) * wl.qo_bytes())
                                          / (sum(attn_ms) / 1e3) / 1e9, 2),
            "attention_frac_of_hbm_peak": round((sum(kv_t) + len(timed) * wl.qo_bytes())
                                                / (sum(attn_ms) / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "note": ("two kernels per step (the shared pass and the stream pass over the "
                     "private blocks in one launch, then the merge); roofline above is that "
                     "launch over every unique byte" if one_launch else
                     "three kernels per step (shared pass, stream pass over the private blocks, "
                     "merge); roofline above is the stream pass over the private bytes"),
        }
    if wl.beam:
        # copy-on-write copies: both caches, every kv head, read + written
        pair_bytes = 4 * wl.Hkv * wl.hd * 16 * wl.eb
        copied = sum(wl.cows[k] for k in timed) * pair_bytes
        res["cow_copy"] = {
            "kernel": ("stage_copy_kernel (the step's staging upload and its copies in one "
                       "launch, pkv_engine_beam_step)" if fused_copy else
                       "copy_blocks_kernel (pkv_copy_blocks)"),
            "pairs_per_step": round(float(np.mean(wl.cows)), 2),
            "bytes_per_pair": pair_bytes,
            "ms_per_step": round(float(np.mean(copy_ms)), 4),
            "achieved_gbs": round(copied / (sum(copy_ms) / 1e3) / 1e9, 2) if copied else None,
            "note": ("measured between HIP events around the launch (includes its launch gap"
                     + ("; and the staging upload, so achieved_gbs is a lower bound)"
                        if fused_copy else ")")),
            "pairs_every_launch": [int(c) for c in wl.cows_all if c],
        }
    # the best of a few wave counts (the probe keeps four tiles in flight per wave; fewer,
    # fuller waves read fastest on this part)
    runs = [bandwidth_probe(torch, pkv, w) for w in (1024, 2048, 4096)]
    probe = {"bytes_per_launch": runs[0]["bytes_per_launch"]}
    for pat in ("sequential_4k_tiles", "random_4k_tiles"):
        best = max(runs, key=lambda r: r[f"{pat}_gbs"])
        probe[f"{pat}_gbs"] = best[f"{pat}_gbs"]
        probe[f"{pat}_waves"] = best["waves"]
    probe["stream_frac_of_random_probe"] = round(achieved / probe["random_4k_tiles_gbs"], 4)
    res["attainable_probe"] = probe
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, torch, W, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
