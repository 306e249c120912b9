"""KV-cache memory accounting: contiguous preallocation versus paged blocks.

Test infrastructure only (see the package docstring).

From the pages:
* [P1] §一 "問題一：內部碎片": a framework that reserves the maximum sequence length up front
  (2048 tokens) for every request wastes whatever the request does not use; a request of
  100 tokens leaves 1948 of its 2048 slots idle (95%).
* [P3] §1.1 and §3.1: the same with 200 tokens (90% waste), and three requests of 200, 500
  and 1000 tokens each holding 2048 slots.
* [P1] §二 "內部碎片": with 16-token blocks taken on demand only a sequence's last block can be
  partly empty, so at most one block per sequence is wasted.
* [P1] §二 "解決三大問題" / [P2] "共享和复用": shared blocks hold one copy of tokens that
  several sequences use.

Definitions (ours, the plain reading of the above):
* contiguous: every request holds ``max_len`` slots; used = its length; utilisation =
  sum(lengths) / (requests * max_len);
* paged: the blocks in use are the distinct blocks named by the sequences' tables (first
  ceil(n/bs) entries); a block's filled slots are the most tokens any sequence keeps in it
  (owners of a shared block hold the same tokens there); utilisation = filled slots /
  (blocks in use * bs). Logical tokens = sum of sequence lengths (a shared token counts once
  per sequence).
"""

import numpy as np


def contiguous_usage(lengths, max_len):
    """(reserved slots, used slots, utilisation) when every request reserves max_len slots."""
    lengths = [int(n) for n in lengths]
    assert all(0 <= n <= max_len for n in lengths), "a request longer than its reservation"
    reserved = len(lengths) * int(max_len)
    used = sum(lengths)
    return reserved, used, (used / reserved if reserved else 0.0)


def paged_usage(tables, lengths, bs):
    """Accounting of a paged cache from its block tables.

    Returns dict(sequences, logical_tokens, blocks_in_use, slots_filled, utilisation)."""
    fill = {}
    logical = 0
    for row, n in zip(tables, lengths):
        n = int(n)
        logical += n
        for j in range(-(-n // bs)):
            b = int(row[j])
            fill[b] = max(fill.get(b, 0), min(bs, n - j * bs))
    blocks = len(fill)
    filled = sum(fill.values())
    return dict(sequences=len(lengths), logical_tokens=logical, blocks_in_use=blocks,
                slots_filled=filled, utilisation=(filled / (blocks * bs) if blocks else 0.0))
