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
  count drops to zero.  Only whole blocks are shared between requests, so a
  shared prefix must end on a block boundary (page "PagedAttention 与连续批处
  理…", advice section); a forked sequence (beam search, section 2.3) shares
  its parent's last, partial block too;
* writing into a shared block first copies it to a private block (copy-on-
  write; page "vLLM的诞生背景…", limitations paragraph), and a sequence's
  blocks can be swapped out to a host pool and back (page "PagedAttention 与
  连续批处理…", section "PagedAttention：把显存做成虚拟内存").  The manager only
  records these copies as (source block, destination block) pairs;
  paged_kv_block_copy moves the bytes.
"""

from typing import Dict, List, Tuple

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
        self._copies: List[Tuple[int, int]] = []
        self._swapped: set = set()  # sequences whose table holds host blocks

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

    def _resident(self, seq: int) -> None:
        """A swapped-out sequence's table holds host block ids: nothing but
        swap_in and finish(seq, host) may touch it."""
        if seq in self._swapped:
            raise ValueError(f"sequence {seq} is swapped out; swap it in first")

    def append_slot(self, seq: int) -> int:
        """Reserve the slot of the sequence's next token; returns the flat slot
        id (physical block * block_size + offset)."""
        self._resident(seq)
        n = self._lens[seq]
        table = self._tables[seq]
        if n % self.block_size == 0:
            table.append(self.allocate())
        j = n // self.block_size
        b = table[j]
        if self.ref_count[b] > 1:
            # copy-on-write: the sequence gets a private copy of the block
            nb = self.allocate()
            self._copies.append((b, nb))
            self.ref_count[b] -= 1
            table[j] = nb
            b = nb
        self._lens[seq] = n + 1
        return b * self.block_size + n % self.block_size

    def fork(self, src: int, dst: int) -> None:
        """dst becomes a copy of src sharing every block, the partial last one
        included; the first write into a shared block copies it."""
        self._resident(src)
        if dst in self._tables:
            raise ValueError(f"sequence {dst} exists")
        self._tables[dst] = []
        for b in self._tables[src]:
            self.ref_count[b] += 1
            self._tables[dst].append(b)
        self._lens[dst] = self._lens[src]

    def take_copies(self) -> np.ndarray:
        """Pending copy-on-write pairs as int32 [n][2] (source, destination),
        to run through paged_kv_block_copy before the write; clears them."""
        out = np.array(self._copies, dtype=np.int32).reshape(-1, 2)
        self._copies = []
        return out

    def swap_out(self, seq: int, host: "BlockManager") -> np.ndarray:
        """Move seq's blocks to host blocks of the host pool's manager; returns
        the (device block, host block) pairs to copy before the device blocks
        are reused.  Only sequences with no shared block can be swapped."""
        self._resident(seq)
        table = self._tables[seq]
        if any(self.ref_count[b] > 1 for b in table):
            raise ValueError("a sequence with shared blocks cannot be swapped out")
        if host.num_free < len(table):
            raise OutOfBlocks("host pool exhausted")
        pairs = []
        for j, b in enumerate(table):
            hb = host.allocate()
            pairs.append((b, hb))
            self.free(b)
            table[j] = hb
        self._swapped.add(seq)
        return np.array(pairs, dtype=np.int32).reshape(-1, 2)

    def swap_in(self, seq: int, host: "BlockManager") -> np.ndarray:
        """Bring a swapped-out sequence back into device blocks; returns the
        (host block, device block) pairs to copy."""
        if seq not in self._swapped:
            raise ValueError(f"sequence {seq} is not swapped out")
        table = self._tables[seq]
        if self.num_free < len(table):
            raise OutOfBlocks("block pool exhausted")
        pairs = []
        for j, hb in enumerate(table):
            b = self.allocate()
            pairs.append((hb, b))
            host.free(hb)
            table[j] = b
        self._swapped.discard(seq)
        return np.array(pairs, dtype=np.int32).reshape(-1, 2)

    def share_prefix(self, src: int, dst: int, num_blocks: int) -> None:
        """Give dst the first num_blocks blocks of src (whole, full blocks)."""
        self._resident(src)
        self._resident(dst)
        if self._tables[dst]:
            raise ValueError("destination must be empty")
        if num_blocks * self.block_size > self._lens[src]:
            raise ValueError("only full blocks can be shared")
        for b in self._tables[src][:num_blocks]:
            self.ref_count[b] += 1
            self._tables[dst].append(b)
        self._lens[dst] = num_blocks * self.block_size

    def finish(self, seq: int, host: "BlockManager" = None) -> None:
        """Release the sequence's blocks.  A swapped-out sequence holds host
        blocks: they go back to the host pool's manager, which must be given."""
        if seq in self._swapped:
            if host is None:
                raise ValueError(f"sequence {seq} is swapped out: finish it with its host manager")
            for hb in self._tables.pop(seq):
                host.free(hb)
            self._swapped.discard(seq)
        else:
            for b in self._tables.pop(seq):
                self.free(b)
        del self._lens[seq]

    # ---------------------------------------------------------------- views
    def block_tables(self, seqs, max_blocks: int, fill: int = 0) -> np.ndarray:
        out = np.full((len(seqs), max_blocks), fill, dtype=np.int32)
        for i, s in enumerate(seqs):
            self._resident(s)
            t = self._tables[s]
            out[i, :len(t)] = t
        return out

    def context_lens(self, seqs) -> np.ndarray:
        return np.array([self._lens[s] for s in seqs], dtype=np.int32)
