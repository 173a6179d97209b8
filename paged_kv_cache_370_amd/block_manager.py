"""Host-side bookkeeping of the block pool: free list, reference counts, per-
sequence block tables and slot ids.  Pure Python; no device work.

What it follows:
* one central manager owns the pre-allocated pool and every request holds a
  block table (dpshk.com PagedAttention article "企业官网建设流程全解析",
  sections 3.1 and 3.2: central BlockManager, pool allocated once);
* logical block j of a sequence maps to a physical block (section 2.1; page
  "vLLM的诞生背景…", section "PagedAttention的破局思路");
* blocks are allocated on demand as a sequence grows and returned when it
  finishes (page "PagedAttention 与连续批处理…", section "PagedAttention：把显存
  做成虚拟内存");
* sharing a block bumps its reference count and puts the same physical block
  in the other table (section 2.3); a block returns to the free list when its
  count drops to zero.  Only whole blocks are shared, so a shared prefix must
  end on a block boundary (page "PagedAttention 与连续批处理…", advice section).
"""

from typing import Dict, List

import numpy as np


class OutOfBlocks(RuntimeError):
    pass


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.ref_count = np.zeros(num_blocks, dtype=np.int64)
        self._free: List[int] = list(range(num_blocks - 1, -1, -1))
        self._tables: Dict[int, List[int]] = {}
        self._lens: Dict[int, int] = {}

    # --------------------------------------------------------------- blocks
    @property
    def num_free(self) -> int:
        return len(self._free)

    def allocate(self) -> int:
        if not self._free:
            raise OutOfBlocks("block pool exhausted")
        b = self._free.pop()
        self.ref_count[b] = 1
        return b

    def free(self, b: int) -> None:
        if self.ref_count[b] <= 0:
            raise ValueError(f"block {b} is not allocated")
        self.ref_count[b] -= 1
        if self.ref_count[b] == 0:
            self._free.append(b)

    # ------------------------------------------------------------ sequences
    def add_sequence(self, seq: int) -> None:
        if seq in self._tables:
            raise ValueError(f"sequence {seq} exists")
        self._tables[seq] = []
        self._lens[seq] = 0

    def table(self, seq: int) -> List[int]:
        return list(self._tables[seq])

    def length(self, seq: int) -> int:
        return self._lens[seq]

    def append_slot(self, seq: int) -> int:
        """Reserve the slot of the sequence's next token; returns the flat slot
        id (physical block * block_size + offset)."""
        n = self._lens[seq]
        table = self._tables[seq]
        if n % self.block_size == 0:
            table.append(self.allocate())
        b = table[n // self.block_size]
        if self.ref_count[b] > 1:
            raise ValueError("appending into a shared block needs copy-on-write")
        self._lens[seq] = n + 1
        return b * self.block_size + n % self.block_size

    def share_prefix(self, src: int, dst: int, num_blocks: int) -> None:
        """Give dst the first num_blocks blocks of src (whole, full blocks)."""
        if self._tables[dst]:
            raise ValueError("destination must be empty")
        if num_blocks * self.block_size > self._lens[src]:
            raise ValueError("only full blocks can be shared")
        for b in self._tables[src][:num_blocks]:
            self.ref_count[b] += 1
            self._tables[dst].append(b)
        self._lens[dst] = num_blocks * self.block_size

    def finish(self, seq: int) -> None:
        for b in self._tables.pop(seq):
            self.free(b)
        del self._lens[seq]

    # ---------------------------------------------------------------- views
    def block_tables(self, seqs, max_blocks: int, fill: int = 0) -> np.ndarray:
        out = np.full((len(seqs), max_blocks), fill, dtype=np.int32)
        for i, s in enumerate(seqs):
            t = self._tables[s]
            out[i, :len(t)] = t
        return out

    def context_lens(self, seqs) -> np.ndarray:
        return np.array([self._lens[s] for s in seqs], dtype=np.int32)
