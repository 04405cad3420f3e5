"""Host-side block manager: demand allocation, fork, copy-on-write, free.

Builds the block tables, slot mappings and copy lists that the shared-prefix
workloads hand to the kernels.  No attention arithmetic lives here.

Rules followed:
  * a new physical block is taken only when the sequence's last block is full
    (Lecture 7 "KV Cache Management" §4.1; Lecture 16 "LLM Serving (1)" §3.3;
    Month 2 "PagedAttention" §6.4, blocks needed = ceil(tokens / block size));
  * fork makes the children's tables point at the parent's physical blocks and
    raises each block's reference count (Lecture 7 §5.1 step 1);
  * before a sequence writes into a block whose count is above one, the block
    is copied to a fresh one and the old block's count drops by one; a writer
    that finds the count at one writes in place (Lecture 7 §5.1 step 2 and
    exercise 4; Lecture 16 §3.5);
  * free drops every count by one and returns blocks that reach zero to the
    free list (Lecture 7 §5.1 step 3).
The kernels only ever see the resulting lists of physical block ids
(Lecture 7 §5.3).
"""
from __future__ import annotations

from collections import deque
from typing import Dict, Iterable, List, Optional, Tuple


class OutOfBlocks(RuntimeError):
    pass


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Iterable[int]] = None):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of the block ids")
        self.free: deque = deque(order)
        self.refcount: List[int] = [0] * self.num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lengths: Dict[int, int] = {}
        self._next_seq = 0
        self.copies: List[Tuple[int, int]] = []   # pending (src, dst) copies, in order

    # -- allocation -------------------------------------------------------
    def _take(self) -> int:
        if not self.free:
            raise OutOfBlocks("no free physical block")
        b = self.free.popleft()
        assert self.refcount[b] == 0
        self.refcount[b] = 1
        return b

    def _release(self, b: int) -> None:
        assert self.refcount[b] > 0
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            self.free.append(b)

    # -- the three operations -------------------------------------------------
    def new_sequence(self) -> int:
        s = self._next_seq
        self._next_seq += 1
        self.tables[s] = []
        self.lengths[s] = 0
        return s

    def append(self, seq: int, n_tokens: int = 1) -> List[int]:
        """Append n_tokens to seq; returns their slot ids (block * block_size + offset).

        Copy-on-write copies this causes are appended to ``self.copies``.
        """
        slots = []
        table = self.tables[seq]
        for _ in range(n_tokens):
            pos = self.lengths[seq]
            off = pos % self.block_size
            if off == 0:
                table.append(self._take())
            else:
                last = table[-1]
                if self.refcount[last] > 1:
                    fresh = self._take()
                    self.copies.append((last, fresh))
                    self.refcount[last] -= 1
                    table[-1] = fresh
            slots.append(table[-1] * self.block_size + off)
            self.lengths[seq] = pos + 1
        return slots

    def fork(self, seq: int, n: int) -> List[int]:
        """Turn seq into n sequences that share its blocks: seq itself plus n-1 children."""
        out = [seq]
        for _ in range(n - 1):
            c = self.new_sequence()
            self.tables[c] = list(self.tables[seq])
            self.lengths[c] = self.lengths[seq]
            for b in self.tables[c]:
                self.refcount[b] += 1
            out.append(c)
        return out

    def free_sequence(self, seq: int) -> None:
        for b in self.tables.pop(seq):
            self._release(b)
        self.lengths.pop(seq)

    # -- views ---------------------------------------------------------------
    def take_copies(self) -> List[Tuple[int, int]]:
        c, self.copies = self.copies, []
        return c

    def blocks_in_use(self) -> int:
        return sum(1 for r in self.refcount if r > 0)

    def table_array(self, seqs: List[int], width: Optional[int] = None):
        import numpy as np
        w = max(len(self.tables[s]) for s in seqs) if width is None else width
        t = np.full((len(seqs), max(w, 1)), -1, dtype=np.int32)
        for i, s in enumerate(seqs):
            t[i, :len(self.tables[s])] = self.tables[s]
        return t
