"""Continuous-batching replay: the scheduler drives the three kernels step by
step over a stream of synthetic requests.

Each step: the scheduler plans (decodes first, then prefill chunks under the
token budget); blocks of requests preempted in this step go to pinned host
pools and blocks of resumed ones come back (pa_swap_blocks); any
copy-on-write copies run (pa_copy_blocks); the step's new
K/V rows go into the cache (pa_reshape_and_cache); the chunks attend their
paged history (pa_prefill_chunk) and the decodes theirs (pa_decode); finished
requests return their blocks.  Request lengths, q rows and new K/V rows are
synthetic and seeded: lengths stand in for end-of-sequence, N(0,1) rows for
the projections of a model.

With a system prompt configured, requests carry token ids and are admitted
through the prefix cache: a request whose prompt starts with cached full
blocks reuses them and prefills only the rest.  The block size of the pools
is a parameter (8, 16, 32 or 64 tokens).

Sources, cited by page title and section: "Lecture 33: KV Cache memory
management -- PagedAttention, Continuous Batching and Chunked Prefill" §3.2
(iteration-level scheduling), §4.2-4.4 (chunked prefill under one token
budget), §5.2 (preemption by swapping), §6.1-6.3 (prefix caching), §2.2 and
appendix Q3 (block size); "PagedAttention: managing the KV cache like virtual
memory" §3.3 (blocks taken as sequences grow, returned as they end), §3.4
(prefix sharing by block hashes).
"""
from __future__ import annotations

import math
import time
from dataclasses import dataclass
from typing import List, Optional, Tuple

import numpy as np
import torch

from . import binding
from .block_manager import BlockPool
from .scheduler import Scheduler, StepPlan, synthetic_requests

_TORCH = {"bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}


@dataclass
class ReplayConfig:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    cache_dtype: str          # "bf16" or "fp8"
    num_blocks: int
    budget: int               # tokens per step (decodes + prefill chunks)
    num_requests: int
    prompt: Tuple[int, int]   # uniform prompt lengths, closed range
    output: Tuple[int, int]   # uniform output lengths, closed range
    seed: int
    kv_scale: float = 1.0
    decode_reserve: bool = True  # False: admit greedily, preempt by swapping
    host_blocks: int = 0         # blocks of the pinned host pools (swap space)
    block_size: int = 16         # tokens per block: 8, 16, 32 or 64
    system_prompt: int = 0       # > 0: requests carry token ids, and a fraction
    share: float = 0.0           #   `share` of them starts with one system prompt
                                 #   of this many tokens (prefix caching)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def width(self) -> int:
        return -(-(self.system_prompt + self.prompt[1] + self.output[1]) // self.block_size)

    @property
    def kv_bytes_per_token(self) -> int:
        return 2 * self.num_kv_heads * self.head_dim * (1 if self.cache_dtype == "fp8" else 2)


REPLAYS = {
    # one attention layer of a Qwen2.5-7B-shaped model serving 512 requests
    "replay_qwen7b": ReplayConfig("replay_qwen7b", 28, 4, 128, "bf16", num_blocks=40000,
                                  budget=2048, num_requests=512, prompt=(64, 3000),
                                  output=(16, 256), seed=157010),
    # the same, with a 1,024-token system prompt ahead of 3 in 4 prompts, served
    # from the prefix cache after its first prefill ([L33] §6.1)
    "replay_qwen7b_prefix": ReplayConfig("replay_qwen7b_prefix", 28, 4, 128, "bf16",
                                         num_blocks=40000, budget=2048, num_requests=512,
                                         prompt=(64, 3000), output=(16, 256), seed=157011,
                                         system_prompt=1024, share=0.75),
}


@dataclass
class StepRecord:
    plan: StepPlan
    gpu_ms: float             # kernels of the step, HIP events on the stream
    decode_ctx_tokens: int    # tokens the decodes attended
    prefill_rows: int


class Replay:
    """Runs a ReplayConfig on one device.  ``keep`` keeps each step's device
    inputs and outputs on the last record (for checks against the oracle)."""

    def __init__(self, cfg: ReplayConfig, device: torch.device, keep: bool = False):
        binding.load()
        self.cfg = cfg
        self.dev = device
        self.keep = keep
        self.pool = BlockPool(cfg.num_blocks, seed=cfg.seed, block_size=cfg.block_size)
        self.host_pool = (BlockPool(cfg.host_blocks, seed=cfg.seed + 1, block_size=cfg.block_size)
                          if cfg.host_blocks else None)
        self.sched = Scheduler(self.pool, cfg.budget, decode_reserve=cfg.decode_reserve,
                               host_pool=self.host_pool)
        for r in synthetic_requests(cfg.num_requests, cfg.seed, cfg.prompt, cfg.output,
                                    system_prompt=cfg.system_prompt, share=cfg.share):
            self.sched.add(r)
        g = torch.Generator(device=device)
        g.manual_seed(cfg.seed)
        shape = (cfg.num_blocks, cfg.block_size, cfg.num_kv_heads, cfg.head_dim)
        cdt = _TORCH[cfg.cache_dtype]
        # recycled blocks hold stale rows, never zeros: start from random bits
        self.k_cache = torch.randn(shape, generator=g, device=device).to(cdt)
        self.v_cache = torch.randn(shape, generator=g, device=device).to(cdt)
        self.k_host = self.v_host = None
        if cfg.host_blocks:
            hshape = (cfg.host_blocks,) + shape[1:]
            self.k_host = torch.empty(hshape, dtype=cdt).pin_memory()
            self.v_host = torch.empty(hshape, dtype=cdt).pin_memory()
        # step rows are slices of fixed random buffers (budget rows each)
        B = cfg.budget
        self.q_buf = torch.randn((B, cfg.num_q_heads, cfg.head_dim), generator=g,
                                 device=device).to(torch.bfloat16)
        self.k_buf = torch.randn((B, cfg.num_kv_heads, cfg.head_dim), generator=g,
                                 device=device).to(torch.bfloat16)
        self.v_buf = torch.randn((B, cfg.num_kv_heads, cfg.head_dim), generator=g,
                                 device=device).to(torch.bfloat16)
        self.out_buf = torch.empty((B, cfg.num_q_heads, cfg.head_dim), dtype=torch.float32,
                                   device=device)
        self.records: List[StepRecord] = []
        self.last: Optional[dict] = None

    @property
    def done(self) -> bool:
        return self.sched.idle

    def step(self) -> StepRecord:
        cfg, dev = self.cfg, self.dev
        plan = self.sched.schedule()
        if plan.num_tokens == 0:
            raise RuntimeError("a step with no work: every waiting prompt is blocked")
        to_dev = lambda a: torch.from_numpy(a).to(dev, non_blocking=False)
        sm = to_dev(plan.slot_mapping())
        n_pre = sum(c.n for c in plan.chunks)
        D = len(plan.decodes)
        T = n_pre + D
        pre = dec = None
        if plan.chunks:
            bt, qs, ctx = plan.prefill_inputs(cfg.width)
            pre = dict(bt=to_dev(bt), qs=to_dev(qs), ctx=to_dev(ctx), host=(bt, qs, ctx))
        if D:
            bt, lens = plan.decode_inputs(cfg.width)
            dec = dict(bt=to_dev(bt), lens=to_dev(lens), host=(bt, lens))
        cow = to_dev(np.asarray(plan.cow, dtype=np.int64).reshape(-1, 2)) if plan.cow else None
        pairs = lambda x: to_dev(np.asarray(x, dtype=np.int64).reshape(-1, 2)) if x else None
        s_out, s_in = pairs(plan.swap_out), pairs(plan.swap_in)
        q = self.q_buf[:T]
        out = self.out_buf[:T]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        if s_out is not None:  # before anything reuses the freed device blocks
            binding.swap_blocks(self.k_cache, self.v_cache, self.k_host, self.v_host, s_out)
        if s_in is not None:
            binding.swap_blocks(self.k_host, self.v_host, self.k_cache, self.v_cache, s_in)
        if cow is not None:
            binding.copy_blocks(self.k_cache, self.v_cache, cow)
        binding.reshape_and_cache(self.k_buf[:T], self.v_buf[:T], self.k_cache, self.v_cache, sm,
                                  kv_scale=cfg.kv_scale)
        if pre is not None:
            binding.prefill_chunk(out[:n_pre], q[:n_pre], self.k_cache, self.v_cache, pre["bt"],
                                  pre["qs"], pre["ctx"], cfg.scale, kv_scale=cfg.kv_scale)
        if dec is not None:
            binding.decode(out[n_pre:], q[n_pre:], self.k_cache, self.v_cache, dec["bt"],
                           dec["lens"], cfg.scale, kv_scale=cfg.kv_scale)
        e1.record()
        torch.cuda.synchronize()
        rec = StepRecord(plan, e0.elapsed_time(e1),
                         int(dec["host"][1].sum()) if dec is not None else 0, n_pre)
        if self.keep:
            self.last = dict(plan=plan, n_pre=n_pre, D=D, T=T, pre=pre, dec=dec,
                             q=q, out=out.clone(), k=self.k_buf[:T], v=self.v_buf[:T])
        self.sched.complete(plan)
        self.records.append(rec)
        return rec


def run(cfg: ReplayConfig, device: torch.device, max_steps: Optional[int] = None) -> dict:
    """Run the replay to the end (or max_steps) and summarise the steady state:
    the steps from the first with at least half the largest decode count to
    the last such step (the ramp-up and the drain excluded)."""
    rp = Replay(cfg, device)
    t0 = time.perf_counter()
    while not rp.done and (max_steps is None or len(rp.records) < max_steps):
        rp.step()
    wall = time.perf_counter() - t0
    recs = rp.records
    D = np.array([len(r.plan.decodes) for r in recs])
    idx = np.nonzero(D >= D.max() / 2)[0]
    ss = recs[idx[0]:idx[-1] + 1]
    gpu_s = sum(r.gpu_ms for r in ss) * 1e-3
    toks = sum(r.plan.num_tokens for r in ss)
    kv = sum(r.decode_ctx_tokens for r in ss) * cfg.kv_bytes_per_token
    fin = rp.sched.finished
    prompt_tokens = sum(r.prompt_len for r in fin)
    saved = sum(r.hit_tokens for r in fin)
    return dict(steps=len(recs), steady_steps=len(ss), finished=len(fin),
                preemptions=rp.sched.preemptions, block_size=cfg.block_size,
                prompt_tokens=prompt_tokens, prefill_tokens_saved=saved,
                prefill_saved_frac=round(saved / max(prompt_tokens, 1), 4),
                wall_s=round(wall, 2),
                gpu_ms_per_step=round(gpu_s * 1e3 / len(ss), 4),
                tokens_per_s_gpu=round(toks / gpu_s, 1),
                decode_kv_gbs=round(kv / gpu_s / 1e9, 2),
                mean_decodes=round(float(D[idx[0]:idx[-1] + 1].mean()), 1),
                mean_tokens_per_step=round(toks / len(ss), 1))
