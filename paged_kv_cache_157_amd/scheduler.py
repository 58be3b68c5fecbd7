"""Iteration-level scheduler with a unified token budget (host side).

Every step re-forms the batch: requests that finished in the previous step
have left and returned their blocks, and the step's budget of tokens is
handed out first to the running decodes (one token each), then, in arrival
order, to prompts that still need prefill, each taking
min(tokens it still needs, budget left) as one chunk.  A prompt whose last
chunk runs produces its first output token in that step and decodes from the
next step on; a request leaves at the end of the step that produced its last
output token.  The scheduler only plans: it emits slots, tables and lengths
for the cache write, the chunked prefill and the decode, and the caller runs
them.

Sources, cited by page title and section:
  [L33] "Lecture 33: KV Cache memory management -- PagedAttention, Continuous
        Batching and Chunked Prefill": §3.2 (a finished request leaves at the
        end of its step and a waiting one joins the next), §3.3 (blocks
        returned by a finished request serve the next admission), §4.2 (a long
        prompt runs as a series of chunks, each attending to the earlier ones
        through the cache), §4.3 (one token budget for prefill and decode
        alike), §4.4 (decodes first, one token each; the rest of the budget
        cut into prefill chunks).
        §5.1-5.2 (when a decode finds no free block, the youngest running
        request is preempted: its blocks go to host memory over PCIe and come
        back when there is room).
  [VM]  "PagedAttention: managing the KV cache like virtual memory": §3.3
        (blocks are taken as a sequence grows and returned when it ends).

Prefix caching ([VM] §3.4-3.5; [L33] §6.2-6.3): a request that carries its
prompt's token ids is admitted through the block manager's cached
allocation, which reuses the cached blocks of its longest prefix of full
blocks (a shared system prompt, a conversation's earlier turns), so that only
the missed tokens are prefilled; once its prompt has been prefilled, its full
blocks are registered as cached for later requests.  Requests without token
ids grow their tables chunk by chunk.  The block size is the pool's.

Two admission policies: with ``decode_reserve`` (the default) a prefill chunk
is admitted only while one free block per running decode remains after it,
so the decodes can always grow and nothing is preempted; without it chunks
are admitted while blocks are free, and a decode that then finds none
preempts running requests youngest first, swapping their blocks to the host
pool (recomputation is out of scope: it needs a model).  Swapped requests
resume in the order they were preempted, at the start of a step, once their
blocks fit.  Without a host pool a decode that finds no block raises
PoolExhausted.
"""
from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field
from typing import Deque, List, Optional, Tuple

import numpy as np

from .block_manager import BlockPool, PoolExhausted, SeqTable, swap_in, swap_out


@dataclass
class Request:
    """A request with a synthetic prompt length and output length (the token
    at which it would emit end-of-sequence), and optionally its prompt's token
    ids (for prefix caching)."""
    rid: int
    prompt_len: int
    output_len: int
    token_ids: Optional[List[int]] = None
    table: Optional[SeqTable] = None
    hit_tokens: int = 0   # prompt tokens found in the prefix cache (no prefill)
    prefilled: int = 0    # prompt tokens whose KV is in the cache
    generated: int = 0    # output tokens produced so far
    first_step: int = -1  # step of the first chunk
    done_step: int = -1   # step that produced the last output token
    preempted: int = 0    # times swapped out

    @property
    def decoding(self) -> bool:
        return self.prefilled == self.prompt_len and self.generated < self.output_len


@dataclass
class Chunk:
    """One prefill chunk: prompt positions [start, start + n) of ``req``."""
    req: Request
    start: int
    n: int
    slots: List[int]


@dataclass
class StepPlan:
    step: int
    decodes: List[Request]
    decode_slots: List[int]
    chunks: List[Chunk]
    cow: List[Tuple[int, int]] = field(default_factory=list)
    # block moves to run before anything else in the step: device -> host
    # (preempted requests), then host -> device (resumed ones)
    swap_out: List[Tuple[int, int]] = field(default_factory=list)
    swap_in: List[Tuple[int, int]] = field(default_factory=list)
    preempted: List[Request] = field(default_factory=list)

    @property
    def num_tokens(self) -> int:
        return len(self.decodes) + sum(c.n for c in self.chunks)

    # ---- kernel inputs ---------------------------------------------------
    def slot_mapping(self) -> np.ndarray:
        """Slots of the step's new tokens: prefill chunks (request order, then
        position), then one per decode."""
        out = [s for c in self.chunks for s in c.slots] + list(self.decode_slots)
        return np.asarray(out, dtype=np.int64)

    def decode_inputs(self, width: int) -> Tuple[np.ndarray, np.ndarray]:
        """[D, width] int32 tables (-1 padded) and [D] int32 context lengths of
        the decodes; a decode attends every token up to its own."""
        bt = np.full((len(self.decodes), width), -1, np.int32)
        lens = np.zeros(len(self.decodes), np.int32)
        for i, r in enumerate(self.decodes):
            bt[i, :len(r.table.blocks)] = r.table.blocks
            lens[i] = r.table.num_tokens
        return bt, lens

    def prefill_inputs(self, width: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """Tables, query_start ([R + 1]) and context lengths (chunk included)
        of the chunks, in chunk order."""
        bt = np.full((len(self.chunks), width), -1, np.int32)
        qs = np.zeros(len(self.chunks) + 1, np.int32)
        ctx = np.zeros(len(self.chunks), np.int32)
        for i, c in enumerate(self.chunks):
            bt[i, :len(c.req.table.blocks)] = c.req.table.blocks
            qs[i + 1] = qs[i] + c.n
            ctx[i] = c.start + c.n
        return bt, qs, ctx


class Scheduler:
    """Admits, grows and retires requests under a per-step token budget."""

    def __init__(self, pool: BlockPool, budget: int = 2048, max_chunk: Optional[int] = None,
                 decode_reserve: bool = True, host_pool: Optional[BlockPool] = None):
        if budget <= 0:
            raise ValueError("budget must be positive")
        self.pool = pool
        self.budget = int(budget)
        self.max_chunk = max_chunk
        self.decode_reserve = decode_reserve
        self.host = host_pool
        self.waiting: Deque[Request] = deque()   # arrival order, prefill not finished
        self.running: List[Request] = []         # decoding, oldest first
        self.swapped: Deque[Request] = deque()   # preempted, in preemption order
        self.finished: List[Request] = []
        self.step_no = 0
        self.preemptions = 0

    def add(self, req: Request) -> None:
        if req.prompt_len <= 0 or req.output_len <= 0:
            raise ValueError("prompt and output lengths must be positive")
        self.waiting.append(req)

    @property
    def idle(self) -> bool:
        return not self.waiting and not self.running and not self.swapped

    def schedule(self) -> StepPlan:
        """Plan one step ([L33] §4.4)."""
        left = self.budget
        plan = StepPlan(self.step_no, [], [], [])
        # phase 0: preempted requests come back, in preemption order, while
        # their blocks fit next to one free block per running decode
        while self.swapped:
            r = self.swapped[0]
            if len(r.table.blocks) + len(self.running) + 1 > self.pool.num_free:
                break
            plan.swap_in += swap_in(r.table, self.pool)
            self.swapped.popleft()
            self.running.append(r)
        # phase 1: every running decode gets one token (its newest token's KV
        # is written and it attends everything up to it), oldest first; one
        # that finds no free block preempts the youngest until one is free
        B = self.pool.block_size
        i = 0
        while i < len(self.running) and left > 0:
            r = self.running[i]
            # a new block is taken when the last one is full, or when the token
            # lands in a block other tables share (copy-on-write)
            t = r.table
            needs_block = (t.num_tokens == len(t.blocks) * B or
                           self.pool.ref_cnt(t.blocks[t.num_tokens // B]) > 1)
            while needs_block and self.pool.num_free == 0:
                if self.host is None:
                    raise PoolExhausted("a decode needs a block and nothing can be preempted")
                victim = self.running.pop()  # the youngest
                plan.swap_out += swap_out(victim.table, self.host)
                victim.preempted += 1
                self.preemptions += 1
                self.swapped.append(victim)
                plan.preempted.append(victim)
                if victim is r:
                    break
            if r not in self.running:
                break  # r preempted itself: every older one is served
            slot, cow = r.table.append_token()
            if cow is not None:
                plan.cow.append(cow)
            plan.decodes.append(r)
            plan.decode_slots.append(slot)
            left -= 1
            i += 1
        # phase 2: prefill chunks in arrival order from what is left
        for r in self.waiting:
            if left == 0:
                break
            # with the reserve: keep one free block per running decode, so that
            # every decode can still grow by a block in the next step
            reserve = len(self.running) if self.decode_reserve else 0
            if r.table is None and r.token_ids is not None:
                # admission through the prefix cache: the table covers the whole
                # prompt at once, its cached prefix needs no prefill
                if self.swapped:
                    break  # preempted requests go first
                try:
                    r.table, r.hit_tokens = SeqTable.allocate_cached(self.pool, r.token_ids, reserve)
                except PoolExhausted:
                    break  # no room: this prompt and later ones wait
                r.prefilled = r.hit_tokens
            need = r.prompt_len - r.prefilled
            n = min(need, left)
            if self.max_chunk is not None:
                n = min(n, self.max_chunk)
            if r.token_ids is not None:
                # blocks already reserved for the whole prompt
                slots = [r.table.slot(p) for p in range(r.prefilled, r.prefilled + n)]
                cows = []
            else:
                if r.table is None:
                    r.table = SeqTable(self.pool)
                have = len(r.table.blocks) * B - r.table.num_tokens
                new_blocks = -(-max(0, n - have) // B)
                if (self.swapped and r.prefilled == 0) or new_blocks > self.pool.num_free - reserve:
                    break  # no room, or preempted requests go first: this prompt and later ones wait
                slots, cows = r.table.extend(n)
            plan.cow += cows
            if r.first_step < 0:
                r.first_step = self.step_no
            plan.chunks.append(Chunk(r, r.prefilled, n, slots))
            left -= n
        if plan.num_tokens == 0 and not self.idle:
            raise PoolExhausted("no request can make progress: the pool is held by waiting prompts "
                                "and preempted requests")
        return plan

    def complete(self, plan: StepPlan) -> List[Request]:
        """Account for a step that ran: prompts whose last chunk ran produce
        their first output token and start decoding; every decode produces
        one token; requests that produced their last token leave and return
        their blocks ([L33] §3.2).  Returns the requests that finished."""
        done = []
        for c in plan.chunks:
            r = c.req
            r.prefilled += c.n
            if r.prefilled == r.prompt_len:
                if r.token_ids is not None:
                    # the prompt's KV is in the pool: its full blocks become
                    # reusable prefix blocks
                    r.table.cache_full_blocks()
                r.generated = 1
                self.waiting.remove(r)
                if r.generated == r.output_len:
                    done.append(r)
                else:
                    self.running.append(r)
        for r in plan.decodes:
            r.generated += 1
            if r.generated == r.output_len:
                done.append(r)
                self.running.remove(r)
        for r in done:
            r.done_step = self.step_no
            r.table.release()
            self.finished.append(r)
        self.step_no += 1
        return done


def synthetic_requests(n: int, seed: int, prompt: Tuple[int, int] = (64, 3000),
                       output: Tuple[int, int] = (16, 256), system_prompt: int = 0,
                       share: float = 0.0, vocab: int = 32000) -> List[Request]:
    """``n`` requests with prompt and output lengths drawn uniformly from the
    given closed ranges (seeded); lengths stand in for EOS.  With
    ``system_prompt`` > 0 every request carries token ids (random, seeded), and
    a fraction ``share`` of them starts with one common system prompt of that
    many tokens ahead of its own prompt ([L33] §6.1: a long system prompt
    repeated across requests), which the prefix cache serves after the first
    such request has been prefilled."""
    rng = np.random.Generator(np.random.PCG64(seed))
    p = rng.integers(prompt[0], prompt[1], size=n, endpoint=True)
    o = rng.integers(output[0], output[1], size=n, endpoint=True)
    if system_prompt <= 0:
        return [Request(i, int(a), int(b)) for i, (a, b) in enumerate(zip(p, o))]
    system = [int(x) for x in rng.integers(0, vocab, size=system_prompt)]
    out = []
    for i, (a, b) in enumerate(zip(p, o)):
        own = [int(x) for x in rng.integers(0, vocab, size=int(a))]
        ids = (system + own) if rng.random() < share else own
        out.append(Request(i, len(ids), int(b), token_ids=ids))
    return out
