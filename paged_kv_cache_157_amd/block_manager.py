"""Host-side block manager: free queue, reference counts, copy-on-write.

It hands the GPU kernels their integer inputs (block tables, context lengths,
slot mappings); it never touches KV data.

Sources, cited by page title and section:
  [L33] "Lecture 33: KV Cache memory management -- PagedAttention, Continuous
        Batching and Chunked Prefill": §2.2 (block size, block table, the
        token-37 addressing walk-through), §2.4 (ref_cnt, copy-on-write).
  [VM]  "PagedAttention: managing the KV cache like virtual memory": §2 (the
        block life cycle), §3.2 (free queue: allocate from the head, free to
        the tail, both O(1); per-block ref_cnt), §3.3 (growth one block at a
        time; release decrements ref_cnt and frees at zero), §3.4 (shared
        prefix blocks; copy-on-write splits a shared block).

Differences from the pages' own sketches:
  - The free queue starts as a seeded permutation of the block ids, so that
    tables come out scattered across the pool as they do after a long run of
    allocations and frees.  Without a seed it starts in id order.
  - Running out of blocks raises ``PoolExhausted``.  Neither a silent
    overcommit nor a sequence growing without a block is possible.
"""
from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field
from typing import Iterable, List, Optional, Tuple

import numpy as np

BLOCK_SIZE = 16  # tokens per KV block ([L33] §2.2; [VM] §1)


class PoolExhausted(RuntimeError):
    """No free block is left for an allocation."""


class RefCountError(RuntimeError):
    """A block was freed or shared while not owned."""


def slot_of(table: List[int], position: int, block_size: int = BLOCK_SIZE) -> int:
    """Flat slot index of logical token ``position``.

    The logical block is position // block_size, the offset is
    position % block_size, the physical block comes from the table, and the
    slot is physical_block * block_size + offset ([L33] §2.2 walk-through).
    """
    return int(table[position // block_size]) * block_size + position % block_size


class BlockPool:
    """Fixed pool of ``num_blocks`` physical blocks with a FIFO free queue."""

    def __init__(self, num_blocks: int, seed: Optional[int] = None):
        if num_blocks <= 0:
            raise ValueError("num_blocks must be positive")
        self.num_blocks = int(num_blocks)
        order = np.arange(self.num_blocks)
        if seed is not None:
            order = np.random.Generator(np.random.PCG64(seed)).permutation(self.num_blocks)
        self._free = deque(int(b) for b in order)
        self._ref = np.zeros(self.num_blocks, dtype=np.int64)

    # -- queries ---------------------------------------------------------
    @property
    def num_free(self) -> int:
        return len(self._free)

    def ref_cnt(self, block: int) -> int:
        return int(self._ref[block])

    def ref_counts(self) -> np.ndarray:
        return self._ref.copy()

    def free_blocks(self) -> List[int]:
        """The free queue, head first (the order allocations take them)."""
        return list(self._free)

    # -- verbs -------------------------------------------------------------
    def allocate(self, n: int) -> List[int]:
        """Pop ``n`` blocks from the head of the free queue, ref_cnt = 1."""
        if n < 0:
            raise ValueError("n must be >= 0")
        if n > len(self._free):
            raise PoolExhausted(f"need {n} blocks, {len(self._free)} free of {self.num_blocks}")
        out = [self._free.popleft() for _ in range(n)]
        for b in out:
            assert self._ref[b] == 0
            self._ref[b] = 1
        return out

    def share(self, blocks: Iterable[int]) -> None:
        """Another table references these blocks: ref_cnt += 1."""
        for b in blocks:
            if self._ref[b] <= 0:
                raise RefCountError(f"block {b} is free and cannot be shared")
            self._ref[b] += 1

    def free(self, blocks: Iterable[int]) -> None:
        """Drop one reference each; a block reaching 0 goes to the queue tail."""
        for b in blocks:
            if self._ref[b] <= 0:
                raise RefCountError(f"block {b} freed with ref_cnt {self._ref[b]}")
            self._ref[b] -= 1
            if self._ref[b] == 0:
                self._free.append(int(b))


@dataclass
class SeqTable:
    """Block table of one sequence: logical block i lives in ``blocks[i]``."""

    pool: BlockPool
    blocks: List[int] = field(default_factory=list)
    num_tokens: int = 0

    @classmethod
    def allocate(cls, pool: BlockPool, num_tokens: int) -> "SeqTable":
        """Table for a fresh sequence already holding ``num_tokens`` tokens."""
        t = cls(pool)
        t.blocks = pool.allocate(-(-num_tokens // BLOCK_SIZE))
        t.num_tokens = num_tokens
        return t

    @classmethod
    def with_prefix(cls, pool: BlockPool, prefix: List[int], num_tokens: int) -> "SeqTable":
        """Sequence whose first len(prefix) blocks are shared with another table.

        Every shared block must hold at least one of this sequence's tokens.
        The last shared block may be partly filled (a fork, [L33] §2.4); the
        first write into it then goes through copy-on-write.
        """
        if num_tokens <= (len(prefix) - 1) * BLOCK_SIZE:
            raise ValueError("a sequence must reach into every block it shares")
        extra = max(0, -(-num_tokens // BLOCK_SIZE) - len(prefix))
        own = pool.allocate(extra)
        pool.share(prefix)
        return cls(pool, list(prefix) + own, num_tokens)

    def slot(self, position: int) -> int:
        if not 0 <= position < len(self.blocks) * BLOCK_SIZE:
            raise IndexError(f"position {position} is not backed by a block")
        return slot_of(self.blocks, position)

    def append_token(self) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Reserve the slot of the next token.

        Returns ``(slot, cow)``.  A new block is popped when the last one is
        full ([VM] §3.3).  If the token lands in a block that other tables
        also reference, that block is first copied to a private one
        ([L33] §2.4): ``cow = (src_block, dst_block)`` names the copy the
        caller must perform on the device before writing; otherwise None.
        """
        pos = self.num_tokens
        cow = None
        if pos == len(self.blocks) * BLOCK_SIZE:
            self.blocks += self.pool.allocate(1)
        else:
            lb = pos // BLOCK_SIZE
            src = self.blocks[lb]
            if self.pool.ref_cnt(src) > 1:
                dst = self.pool.allocate(1)[0]
                self.pool.free([src])
                self.blocks[lb] = dst
                cow = (src, dst)
        self.num_tokens = pos + 1
        return self.slot(pos), cow

    def release(self) -> None:
        """The sequence finished: every block loses one reference."""
        self.pool.free(self.blocks)
        self.blocks = []
        self.num_tokens = 0

    def waste(self) -> int:
        """Reserved but unused token slots (always < one block)."""
        return len(self.blocks) * BLOCK_SIZE - self.num_tokens


def pack_tables(tables: List[SeqTable], width: int, pad: int = -1) -> np.ndarray:
    """[num_seqs, width] int32 block table; entries past a table's end are ``pad``."""
    out = np.full((len(tables), width), pad, dtype=np.int32)
    for i, t in enumerate(tables):
        if len(t.blocks) > width:
            raise ValueError(f"table {i} has {len(t.blocks)} blocks > width {width}")
        out[i, :len(t.blocks)] = t.blocks
    return out
