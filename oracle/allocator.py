"""Block allocator: allocate on demand, share, copy-on-write, free on finish.

Test infrastructure only (see the package docstring).

From the pages:
* [P1] §三 步驟一: a new request starts with an empty block table; blocks are not reserved up
  front but taken when needed.
* [P1] §三 步驟二/步驟三: tokens are written into the current block while it has room; when it
  is full a new block is taken and the table updated.
* [P1] §三 步驟四: when the request finishes all its blocks are released and may serve others.
* [P1] §二 "解決三大問題" and [P2] "共享和复用": several block tables may point at the same
  physical blocks (common system prompt, shared history, beam candidates).

Where the pages are silent (our reading, the same as the library's documented contract):
* free list = FIFO queue, initially ``free_order`` (default 0..NB-1); take from the front,
  return to the back;
* sharing is counted per physical block (refcount); ``fork`` makes a child that points at all
  of its parent's blocks;
* a sequence appending into a partly filled last block that others still point at first moves
  to a fresh block (copy-on-write) and reports (src, dst) so that the caller copies the data;
* ``free`` walks the sequence's blocks in logical order and returns each block whose count
  reaches zero;
* a batch ``append`` serves sequences in argument order and tokens in order; it checks the
  total number of blocks it needs before changing anything (all-or-nothing).

Automatic prefix caching ([P1] §五 "前綴共享" and §八 "前綴快取": requests with the same
prefix share its KV cache without the caller saying so; [P3] §4.2: a 2000-token system prompt
reused by a later request). Our reading, for full blocks only:
* a full block's content is named by (the node of the block before it, or the root, and the
  block's bs token ids), so a block matches only when its whole prefix matches;
* ``add_seq_tokens`` starts a sequence from a prompt: it shares the longest chain of cached
  full blocks that the prompt begins with, takes fresh blocks for the rest and indexes the
  prompt's new full blocks; ``append_tokens`` is ``append`` with the tokens' ids, and
  indexes blocks that become full. Sequences created or grown without ids are not indexed;
* a freed block keeps its index entry and stays in the free list in FIFO order: a hit takes it
  back out (refcount 1), a fresh allocation that pops it drops the entry (eviction).
"""

from collections import deque


class AllocError(Exception):
    """Raised with one of: INVALID_ARG, OUT_OF_BLOCKS, UNKNOWN_SEQ, SEQ_EXISTS."""

    def __init__(self, code):
        super().__init__(code)
        self.code = code


class BlockAllocator:
    def __init__(self, num_blocks, block_size, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise AllocError("INVALID_ARG")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise AllocError("INVALID_ARG")
        self.num_blocks = num_blocks
        self.bs = block_size
        self.free = deque(order)
        self.ref = [0] * num_blocks
        self.blocks = {}  # seq id -> list of physical blocks, logical order
        self.length = {}  # seq id -> tokens
        # prefix cache: (parent node, token ids) -> node; node -> block; block -> node
        self.index = {}
        self.node_block = {}
        self.node_key = {}
        self.block_node = {}
        self.next_node = 1  # node 0 is the root (the empty prefix)
        self.track = {}     # seq id -> [node of its last indexed full block, pending ids] or None

    # -- [P1] §三 步驟一 ---------------------------------------------------------------
    def add_seq(self, seq):
        if seq in self.blocks:
            raise AllocError("SEQ_EXISTS")
        self.blocks[seq] = []
        self.length[seq] = 0
        self.track[seq] = None

    def _take(self):
        """Pop the free list's front for a fresh allocation (evicting its index entry)."""
        b = self.free.popleft()
        node = self.block_node.pop(b, None)
        if node is not None:
            del self.index[self.node_key.pop(node)]
            del self.node_block[node]
        self.ref[b] = 1
        return b

    def _register(self, parent, ids, block):
        """Index a full block under (parent, ids); returns the node now naming that content
        (an existing one if the same content is already indexed)."""
        key = (parent, tuple(int(t) for t in ids))
        if key in self.index:
            return self.index[key]
        node = self.next_node
        self.next_node += 1
        self.index[key] = node
        self.node_key[node] = key
        self.node_block[node] = block
        self.block_node[block] = node
        return node

    # -- [P1] §三 步驟二/步驟三 ----------------------------------------------------------
    def _needs(self, seq, ntok):
        """(copy-on-write block needed?, new blocks needed) for appending ntok tokens."""
        n = self.length[seq]
        blocks = self.blocks[seq]
        cow = ntok > 0 and n % self.bs != 0 and self.ref[blocks[-1]] > 1
        have = (n + self.bs - 1) // self.bs
        want = (n + ntok + self.bs - 1) // self.bs
        return cow, want - have

    def append(self, seqs, ntok, token_ids=None):
        """Append ntok[k] tokens to seqs[k]. Returns (slots, [(src, dst), ...]).

        token_ids (optional, sum(ntok) ids in argument order): the tokens' ids, so that blocks
        of indexed sequences that become full are indexed too (``append_tokens``)."""
        seqs = list(seqs)
        ntok = [int(t) for t in ntok]
        if len(seqs) != len(ntok) or any(t < 0 for t in ntok) or len(set(seqs)) != len(seqs):
            raise AllocError("INVALID_ARG")
        ids = None
        if token_ids is not None:
            if len(token_ids) != sum(ntok):
                raise AllocError("INVALID_ARG")
            ids, pos = [], 0
            for t in ntok:
                ids.append([int(x) for x in token_ids[pos:pos + t]])
                pos += t
        for s in seqs:
            if s not in self.blocks:
                raise AllocError("UNKNOWN_SEQ")
        # Count what the loop below takes: sharers of a partly filled block that append in
        # this call move off it in argument order, so the last of them finds the refcount back
        # at 1 and writes in place (no copy).
        total, moved = 0, {}
        for s, t in zip(seqs, ntok):
            cow, new = self._needs(s, t)
            if cow:
                b = self.blocks[s][-1]
                cow = self.ref[b] - moved.get(b, 0) > 1
                moved[b] = moved.get(b, 0) + int(cow)
            total += int(cow) + new
        if total > len(self.free):
            raise AllocError("OUT_OF_BLOCKS")
        slots, cows = [], []
        for k, (s, t) in enumerate(zip(seqs, ntok)):
            cow, _ = self._needs(s, t)
            blocks = self.blocks[s]
            if cow:
                src = blocks[-1]
                dst = self._take()
                self.ref[src] -= 1
                blocks[-1] = dst
                cows.append((src, dst))
            for i in range(t):
                n = self.length[s]
                if n % self.bs == 0:  # current block full (or none yet): take a new one
                    blocks.append(self._take())
                slots.append(blocks[n // self.bs] * self.bs + n % self.bs)
                self.length[s] = n + 1
                tr = self.track[s]
                if tr is not None and ids is not None:
                    tr[1].append(ids[k][i])
                    if len(tr[1]) == self.bs:  # the block just filled: index it
                        tr[0] = self._register(tr[0], tr[1], blocks[n // self.bs])
                        tr[1] = []
            if t > 0 and ids is None:
                self.track[s] = None  # tokens of unknown content: no longer indexed
        return slots, cows

    def append_tokens(self, seqs, ntok, token_ids):
        return self.append(seqs, ntok, token_ids)

    # -- automatic prefix caching ------------------------------------------------------
    def add_seq_tokens(self, seq, token_ids):
        """New sequence holding a prompt of len(token_ids) tokens. Shares the longest chain of
        indexed full blocks the prompt begins with. Returns (slots of all prompt tokens,
        tokens found in the cache: a multiple of bs)."""
        if seq in self.blocks:
            raise AllocError("SEQ_EXISTS")
        ids = [int(t) for t in token_ids]
        n, bs = len(ids), self.bs
        parent, hits = 0, []
        for j in range(n // bs):
            node = self.index.get((parent, tuple(ids[j * bs:(j + 1) * bs])))
            if node is None:
                break
            hits.append(self.node_block[node])
            parent = node
        revived = sum(1 for b in hits if self.ref[b] == 0)
        fresh = -(-n // bs) - len(hits)
        if fresh > len(self.free) - revived:
            raise AllocError("OUT_OF_BLOCKS")
        for b in hits:
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1
        blocks = list(hits) + [self._take() for _ in range(fresh)]
        last = parent
        for j in range(len(hits), n // bs):
            last = self._register(last, ids[j * bs:(j + 1) * bs], blocks[j])
        self.blocks[seq] = blocks
        self.length[seq] = n
        self.track[seq] = [last, ids[(n // bs) * bs:]]
        slots = [blocks[t // bs] * bs + t % bs for t in range(n)]
        return slots, len(hits) * bs

    def cached_blocks(self):
        """Blocks whose content is indexed (in use or free)."""
        return len(self.block_node)

    # -- [P1] §二 sharing; [P2] 共享和复用 -----------------------------------------------
    def fork(self, parent, child):
        if parent not in self.blocks:
            raise AllocError("UNKNOWN_SEQ")
        if child in self.blocks:
            raise AllocError("SEQ_EXISTS")
        self.blocks[child] = list(self.blocks[parent])
        self.length[child] = self.length[parent]
        tr = self.track[parent]
        self.track[child] = None if tr is None else [tr[0], list(tr[1])]
        for b in self.blocks[child]:
            self.ref[b] += 1

    # -- [P1] §三 步驟四 ---------------------------------------------------------------
    def free_seq(self, seq):
        if seq not in self.blocks:
            raise AllocError("UNKNOWN_SEQ")
        for b in self.blocks.pop(seq):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.length[seq]
        del self.track[seq]

    # -- queries -----------------------------------------------------------------------
    def tables(self, seqs, max_blocks):
        rows, lens = [], []
        for s in seqs:
            if s not in self.blocks:
                raise AllocError("UNKNOWN_SEQ")
            b = self.blocks[s]
            if len(b) > max_blocks:
                raise AllocError("INVALID_ARG")
            rows.append(list(b) + [-1] * (max_blocks - len(b)))
            lens.append(self.length[s])
        return rows, lens

    def num_free(self):
        return len(self.free)

    def refcount(self, block):
        if not 0 <= block < self.num_blocks:
            return -1
        return self.ref[block]

    def seq_len(self, seq):
        return self.length.get(seq, -1)

    def free_list(self):
        return list(self.free)

    def usage(self):
        """Memory accounting of the live sequences (``utilisation.paged_usage`` over them)."""
        from .utilisation import paged_usage
        seqs = list(self.blocks)
        return paged_usage([self.blocks[s] for s in seqs], [self.length[s] for s in seqs],
                           self.bs)
