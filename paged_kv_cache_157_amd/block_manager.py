"""Host-side block manager: free queue, reference counts, copy-on-write,
prefix caching.

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
        prefix blocks; copy-on-write splits a shared block; a full block is
        identified by a hash of its tokens and its parent block's hash, and a
        request whose prefix hashes are known reuses those blocks), §2 and
        §3.5 (the three block states: free, owned, cached-free).
  [L33] §6.3: the free queue is a doubly linked list so that a cached block
        can be taken out of the middle of it in O(1) on a prefix hit.
  [L33] §5.2, §5.4: preemption by swapping a request's blocks to host memory
        and back; the cost of a round trip is 2 * S * KV_token / B_pcie.

Differences from the pages' own sketches:
  - The free queue starts as a seeded permutation of the block ids, so that
    tables come out scattered across the pool as they do after a long run of
    allocations and frees.  Without a seed it starts in id order.
  - Running out of blocks raises ``PoolExhausted``.  Neither a silent
    overcommit nor a sequence growing without a block is possible.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

BLOCK_SIZE = 16  # default tokens per KV block ([L33] §2.2; [VM] §1); a pool may use 8, 32 or 64


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


def block_hash(parent: Optional[bytes], tokens: Sequence[int]) -> bytes:
    """Identity of a full block for prefix caching: a digest of the parent
    block's hash and the block's token ids ([VM] §3.4), so equal tokens at a
    different position (after a different prefix) give a different hash."""
    h = hashlib.sha256(parent or b"")
    h.update(np.asarray(tokens, dtype=np.int64).tobytes())
    return h.digest()


_NIL = -1


class BlockPool:
    """Fixed pool of ``num_blocks`` physical blocks with a FIFO free queue.

    Every block is in one of three states ([VM] §2, §3.5): free (ref_cnt 0,
    no hash, in the queue), owned (ref_cnt > 0, out of the queue) or cached
    (ref_cnt 0, hash kept, in the queue as an eviction candidate whose KV is
    still valid).  The queue is a doubly linked list over the block ids:
    allocation pops the head, a block whose count drops to zero goes to the
    tail, and a prefix hit unlinks a cached block from anywhere, each O(1).
    """

    def __init__(self, num_blocks: int, seed: Optional[int] = None, block_size: int = BLOCK_SIZE):
        if num_blocks <= 0:
            raise ValueError("num_blocks must be positive")
        if block_size not in (8, 16, 32, 64):
            raise ValueError("block_size must be 8, 16, 32 or 64 tokens")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)  # tokens per block ([L33] §2.2, appendix Q3)
        order = np.arange(self.num_blocks)
        if seed is not None:
            order = np.random.Generator(np.random.PCG64(seed)).permutation(self.num_blocks)
        order = [int(b) for b in order]
        n = self.num_blocks
        self._prev, self._next = [_NIL] * n, [_NIL] * n  # queue links per block id
        for i, b in enumerate(order):
            self._prev[b] = order[i - 1] if i > 0 else _NIL
            self._next[b] = order[i + 1] if i + 1 < n else _NIL
        self._head, self._tail = order[0], order[-1]
        self._in_queue = [True] * n
        self._n_free = n
        self._ref = np.zeros(n, dtype=np.int64)
        self._hash: List[Optional[bytes]] = [None] * n
        self._cached: Dict[bytes, int] = {}

    # -- the queue -------------------------------------------------------
    def _push_tail(self, b: int) -> None:
        self._prev[b], self._next[b] = self._tail, _NIL
        if self._tail == _NIL:
            self._head = b
        else:
            self._next[self._tail] = b
        self._tail = b
        self._in_queue[b] = True
        self._n_free += 1

    def _unlink(self, b: int) -> None:
        p, q = self._prev[b], self._next[b]
        if p == _NIL:
            self._head = q
        else:
            self._next[p] = q
        if q == _NIL:
            self._tail = p
        else:
            self._prev[q] = p
        self._prev[b] = self._next[b] = _NIL
        self._in_queue[b] = False
        self._n_free -= 1

    # -- queries ---------------------------------------------------------
    @property
    def num_free(self) -> int:
        """Blocks in the free queue (free or cached)."""
        return self._n_free

    def ref_cnt(self, block: int) -> int:
        return int(self._ref[block])

    def ref_counts(self) -> np.ndarray:
        return self._ref.copy()

    def free_blocks(self) -> List[int]:
        """The free queue, head first (the order allocations take them)."""
        out, b = [], self._head
        while b != _NIL:
            out.append(b)
            b = self._next[b]
        return out

    def state(self, block: int) -> str:
        """"owned", "cached" or "free" ([VM] §3.5)."""
        if self._ref[block] > 0:
            return "owned"
        return "cached" if self._hash[block] is not None else "free"

    def lookup(self, h: bytes) -> Optional[int]:
        """The block holding the full block with hash ``h``, if any."""
        return self._cached.get(h)

    # -- verbs -------------------------------------------------------------
    def allocate(self, n: int) -> List[int]:
        """Pop ``n`` blocks from the head of the free queue, ref_cnt = 1.  A
        cached block taken this way is evicted: its hash is dropped."""
        if n < 0:
            raise ValueError("n must be >= 0")
        if n > self._n_free:
            raise PoolExhausted(f"need {n} blocks, {self._n_free} free of {self.num_blocks}")
        out = []
        for _ in range(n):
            b = self._head
            self._unlink(b)
            assert self._ref[b] == 0
            h = self._hash[b]
            if h is not None:
                if self._cached.get(h) == b:
                    del self._cached[h]
                self._hash[b] = None
            self._ref[b] = 1
            out.append(b)
        return out

    def touch(self, blocks: Iterable[int]) -> None:
        """A prefix hit: ref_cnt += 1; a cached block leaves the free queue."""
        for b in blocks:
            if self._ref[b] == 0:
                if self._hash[b] is None:
                    raise RefCountError(f"block {b} is free and holds no cached prefix")
                self._unlink(b)
            self._ref[b] += 1

    def cache_block(self, block: int, h: bytes) -> None:
        """Register the hash of an owned full block whose KV has been written.
        If another block already holds that hash, that one stays the cached
        copy and this block is left unregistered."""
        if self._ref[block] <= 0:
            raise RefCountError(f"block {block} is not owned and cannot be cached")
        if h in self._cached or self._hash[block] is not None:
            return
        self._hash[block] = h
        self._cached[h] = block

    def share(self, blocks: Iterable[int]) -> None:
        """Another table references these blocks: ref_cnt += 1."""
        for b in blocks:
            if self._ref[b] <= 0:
                raise RefCountError(f"block {b} is free and cannot be shared")
            self._ref[b] += 1

    def free(self, blocks: Iterable[int]) -> None:
        """Drop one reference each; a block reaching 0 goes to the queue tail
        (keeping its hash, if it has one: owned -> cached)."""
        for b in blocks:
            if self._ref[b] <= 0:
                raise RefCountError(f"block {b} freed with ref_cnt {self._ref[b]}")
            self._ref[b] -= 1
            if self._ref[b] == 0:
                self._push_tail(int(b))


@dataclass
class SeqTable:
    """Block table of one sequence: logical block i lives in ``blocks[i]``."""

    pool: BlockPool
    blocks: List[int] = field(default_factory=list)
    num_tokens: int = 0
    # chained hashes of the full blocks of known token ids (prefix caching)
    hashes: List[bytes] = field(default_factory=list)
    # the token ids, while every token's id is known (prefix caching)
    token_ids: Optional[List[int]] = None

    @property
    def block_size(self) -> int:
        return self.pool.block_size

    @classmethod
    def allocate(cls, pool: BlockPool, num_tokens: int) -> "SeqTable":
        """Table for a fresh sequence already holding ``num_tokens`` tokens."""
        t = cls(pool)
        t.blocks = pool.allocate(-(-num_tokens // pool.block_size))
        t.num_tokens = num_tokens
        return t

    @classmethod
    def with_prefix(cls, pool: BlockPool, prefix: List[int], num_tokens: int) -> "SeqTable":
        """Sequence whose first len(prefix) blocks are shared with another table.

        Every shared block must hold at least one of this sequence's tokens.
        The last shared block may be partly filled (a fork, [L33] §2.4); the
        first write into it then goes through copy-on-write.
        """
        B = pool.block_size
        if num_tokens <= (len(prefix) - 1) * B:
            raise ValueError("a sequence must reach into every block it shares")
        extra = max(0, -(-num_tokens // B) - len(prefix))
        own = pool.allocate(extra)
        pool.share(prefix)
        return cls(pool, list(prefix) + own, num_tokens)

    @classmethod
    def allocate_cached(cls, pool: BlockPool, token_ids: Sequence[int],
                        reserve: int = 0) -> Tuple["SeqTable", int]:
        """Table for a new request with prompt ``token_ids``, reusing cached
        blocks for its longest cached prefix of full blocks ([VM] §3.4;
        [L33] §6.2).  Returns ``(table, hit_tokens)``: the first hit_tokens
        tokens already have their KV in the pool and need no prefill.  A hit
        never covers the whole prompt: at least its last token is computed
        (the step needs an output for it), so a fully cached prompt gives
        back its last full block.  Raises PoolExhausted, with no block taken,
        when the rest does not fit next to ``reserve`` blocks kept free."""
        n = len(token_ids)
        B = pool.block_size
        full = n // B
        hashes, parent = [], None
        for j in range(full):
            parent = block_hash(parent, token_ids[j * B:(j + 1) * B])
            hashes.append(parent)
        hit = []
        for h in hashes:
            b = pool.lookup(h)
            if b is None:
                break
            hit.append(b)
        if hit and len(hit) * B >= n:
            hit.pop()
        need = -(-n // B) - len(hit)
        queued = sum(1 for b in hit if pool.ref_cnt(b) == 0)  # leave the queue on the hit
        if need > pool.num_free - queued - reserve:
            raise PoolExhausted(f"need {need} blocks, {pool.num_free - queued} free after the hit, "
                                f"{reserve} kept")
        pool.touch(hit)
        t = cls(pool, hit + pool.allocate(need), n, hashes, [int(x) for x in token_ids])
        return t, len(hit) * B

    def cache_full_blocks(self) -> None:
        """Register this table's full blocks of known tokens as cached prefix
        blocks, once their KV is in the pool (after the prefill wrote it)."""
        for b, h in zip(self.blocks, self.hashes):
            self.pool.cache_block(b, h)

    def slot(self, position: int) -> int:
        if not 0 <= position < len(self.blocks) * self.block_size:
            raise IndexError(f"position {position} is not backed by a block")
        return slot_of(self.blocks, position, self.block_size)

    def append_token(self, token_id: Optional[int] = None) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Reserve the slot of the next token.

        With the ids of every earlier token known (a table from
        ``allocate_cached``), ``token_id`` extends them, and a block that
        fills gets its chained hash; without it, later blocks are not hashed.

        Returns ``(slot, cow)``.  A new block is popped when the last one is
        full ([VM] §3.3).  If the token lands in a block that other tables
        also reference, that block is first copied to a private one
        ([L33] §2.4): ``cow = (src_block, dst_block)`` names the copy the
        caller must perform on the device before writing; otherwise None.
        """
        pos = self.num_tokens
        B = self.block_size
        cow = None
        if pos == len(self.blocks) * B:
            self.blocks += self.pool.allocate(1)
        else:
            lb = pos // B
            src = self.blocks[lb]
            if self.pool.ref_cnt(src) > 1:
                dst = self.pool.allocate(1)[0]
                self.pool.free([src])
                self.blocks[lb] = dst
                cow = (src, dst)
        self.num_tokens = pos + 1
        if self.token_ids is not None:
            if token_id is None:
                self.token_ids = None
            else:
                self.token_ids.append(int(token_id))
                if self.num_tokens % B == 0 and len(self.hashes) == self.num_tokens // B - 1:
                    parent = self.hashes[-1] if self.hashes else None
                    self.hashes.append(block_hash(parent, self.token_ids[-B:]))
        return self.slot(pos), cow

    def extend(self, n: int) -> Tuple[List[int], List[Tuple[int, int]]]:
        """Reserve the slots of the next ``n`` tokens (a prefill chunk): the
        first goes through ``append_token`` (copy-on-write of a shared last
        block), the rest fill that block and then whole new blocks taken at
        once.  Returns the slots and the copies to perform."""
        if n <= 0:
            return [], []
        if self.token_ids is not None:
            self.token_ids = None  # ids of the new tokens are not known
        first, cow = self.append_token()
        slots = [first]
        pos = self.num_tokens
        B = self.block_size
        room = len(self.blocks) * B - pos
        rest = n - 1
        if rest > room:
            self.blocks += self.pool.allocate(-(-(rest - room) // B))
        for p in range(pos, pos + rest):
            slots.append(slot_of(self.blocks, p, B))
        self.num_tokens = pos + rest
        return slots, [cow] if cow is not None else []

    def release(self) -> None:
        """The sequence finished: every block loses one reference (a cached
        block stays reusable until an allocation evicts it)."""
        self.pool.free(self.blocks)
        self.blocks = []
        self.num_tokens = 0
        self.hashes = []
        self.token_ids = None

    def waste(self) -> int:
        """Reserved but unused token slots (always < one block)."""
        return len(self.blocks) * self.block_size - self.num_tokens


def swap_out(table: SeqTable, host: BlockPool) -> List[Tuple[int, int]]:
    """Preemption by swapping ([L33] §5.2): the table's blocks get blocks of
    the host pool, the device blocks lose this table's reference (a block
    another table shares stays on the device for it), and the table now
    points into the host pool.  Returns the (device, host) block copies to
    run before the freed device blocks are reused."""
    if host.block_size != table.pool.block_size:
        raise ValueError("device and host pools must use the same block size")
    hb = host.allocate(len(table.blocks))
    pairs = list(zip(table.blocks, hb))
    table.pool.free(table.blocks)
    table.pool, table.blocks = host, hb
    return pairs


def swap_in(table: SeqTable, device: BlockPool) -> List[Tuple[int, int]]:
    """Resume a swapped-out table: it gets fresh device blocks (private ones,
    even where its blocks were shared before) and gives its host blocks back.
    Returns the (host, device) block copies to run before it is scheduled."""
    db = device.allocate(len(table.blocks))
    pairs = list(zip(table.blocks, db))
    table.pool.free(table.blocks)
    table.pool, table.blocks = device, db
    table.hashes = []  # the new blocks are not registered as cached prefixes
    return pairs


def swap_time_model(tokens: int, kv_bytes_per_token: int, link_bytes_per_s: float) -> float:
    """Seconds to swap ``tokens`` tokens out and back in over a host link
    ([L33] §5.4): 2 * S * KV_token / B_pcie."""
    return 2.0 * tokens * kv_bytes_per_token / link_bytes_per_s


def pack_tables(tables: List[SeqTable], width: int, pad: int = -1) -> np.ndarray:
    """[num_seqs, width] int32 block table; entries past a table's end are ``pad``."""
    out = np.full((len(tables), width), pad, dtype=np.int32)
    for i, t in enumerate(tables):
        if len(t.blocks) > width:
            raise ValueError(f"table {i} has {len(t.blocks)} blocks > width {width}")
        out[i, :len(t.blocks)] = t.blocks
    return out
