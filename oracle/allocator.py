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

    # -- [P1] §三 步驟一 ---------------------------------------------------------------
    def add_seq(self, seq):
        if seq in self.blocks:
            raise AllocError("SEQ_EXISTS")
        self.blocks[seq] = []
        self.length[seq] = 0

    # -- [P1] §三 步驟二/步驟三 ----------------------------------------------------------
    def _needs(self, seq, ntok):
        """(copy-on-write block needed?, new blocks needed) for appending ntok tokens."""
        n = self.length[seq]
        blocks = self.blocks[seq]
        cow = ntok > 0 and n % self.bs != 0 and self.ref[blocks[-1]] > 1
        have = (n + self.bs - 1) // self.bs
        want = (n + ntok + self.bs - 1) // self.bs
        return cow, want - have

    def append(self, seqs, ntok):
        """Append ntok[k] tokens to seqs[k]. Returns (slots, [(src, dst), ...])."""
        seqs = list(seqs)
        ntok = [int(t) for t in ntok]
        if len(seqs) != len(ntok) or any(t < 0 for t in ntok) or len(set(seqs)) != len(seqs):
            raise AllocError("INVALID_ARG")
        for s in seqs:
            if s not in self.blocks:
                raise AllocError("UNKNOWN_SEQ")
        total = 0
        for s, t in zip(seqs, ntok):
            cow, new = self._needs(s, t)
            total += int(cow) + new
        if total > len(self.free):
            raise AllocError("OUT_OF_BLOCKS")
        slots, cows = [], []
        for s, t in zip(seqs, ntok):
            cow, _ = self._needs(s, t)
            blocks = self.blocks[s]
            if cow:
                src = blocks[-1]
                dst = self.free.popleft()
                self.ref[src] -= 1
                self.ref[dst] = 1
                blocks[-1] = dst
                cows.append((src, dst))
            for _ in range(t):
                n = self.length[s]
                if n % self.bs == 0:  # current block full (or none yet): take a new one
                    b = self.free.popleft()
                    self.ref[b] = 1
                    blocks.append(b)
                slots.append(blocks[n // self.bs] * self.bs + n % self.bs)
                self.length[s] = n + 1
        return slots, cows

    # -- [P1] §二 sharing; [P2] 共享和复用 -----------------------------------------------
    def fork(self, parent, child):
        if parent not in self.blocks:
            raise AllocError("UNKNOWN_SEQ")
        if child in self.blocks:
            raise AllocError("SEQ_EXISTS")
        self.blocks[child] = list(self.blocks[parent])
        self.length[child] = self.length[parent]
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
