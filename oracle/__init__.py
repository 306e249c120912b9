"""CPU oracle for paged decode attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or run anything in
this package: only the test suite, the smoke check and the benchmark's CPU-baseline leg use
it. It shares no code with the HIP library (no kernels, headers, helpers or constants) and
imports nothing from it.

It is a plain, slow, obviously correct restatement of what the pages describe:

* [P1] "vLLM 與 PagedAttention：高吞吐推理的關鍵", §二 (blocks of a fixed number of tokens,
  a block table per request, blocks scattered in memory, shared blocks), §三 steps 一..四
  (empty table at start, write into the current block or take a new one, attend through the
  table, free everything at the end);
* [P2] vLLM overview, "PagedAttention 的核心原理" (logical blocks mapped to physical blocks,
  on-demand allocation, sharing for common prefixes and beam search);
* [P3] "vLLM 与 PagedAttention：大模型高性能推理服务实战", §3.2 (16 tokens per block, one
  block table per request).

The pages state no attention formula; the oracle uses textbook scaled dot-product attention
with max-subtracted softmax, in float64, over each sequence's logical K/V gathered from the
paged cache. Modules:

* ``layout``     -- where token t / dim d of a (block, kv head) tile lives in the caches.
* ``attention``  -- gather + dense attention; partition partials and their log-sum-exp merge.
* ``cache_write``-- the scatter of new tokens into their slots; the copy-on-write block copy.
* ``allocator``  -- FIFO / refcount block allocator (allocate on demand, fork, free, COW).
* ``utilisation``-- memory accounting: contiguous preallocation versus paged blocks.
* ``batching``   -- the continuous-batching step loop (retire, admit + prompt write, decode).
"""

from . import allocator, attention, batching, cache_write, layout, utilisation  # noqa: F401
