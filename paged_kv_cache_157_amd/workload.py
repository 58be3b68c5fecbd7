"""Seeded synthetic workloads shaped like the pages' scenarios.

This module only draws random numbers and asks the block manager for tables
and slots; it holds none of the attention arithmetic.  Tests, the smoke check
and the benchmark use it to feed the same inputs to the HIP library and to
the CPU oracle.

Shapes follow the scenarios the pages discuss: a Qwen2.5-7B-shaped decode
batch (28 query heads, 4 KV heads, head_dim 128), a 13B-shaped MHA batch
(40/40/128) with a shared 1024-token prefix, a skewed long/short mix that
needs split-K partitions, and a chunked-prefill mixed step (a 512-token
chunk over an 8192-token paged history plus 96 decodes), each with
block_size 16.  Values are N(0,1).

Recipe (also what the seeds pin):
  * lengths: numpy PCG64(seed); "uniform in [a, b]" means integers, both
    ends included; lognormal lengths use sigma 1 around the stated median,
    rounded and clipped;
  * tables: a BlockPool whose free queue is a PCG64(seed) permutation of the
    pool, so tables are scattered; sequences allocate in index order;
  * values: torch's generator seeded with the same seed on the target
    device, N(0,1) in fp32, rounded to the storage type (bf16 RNE; fp8
    E4M3FN via torch's saturating-free cast of the clamped x * 1/scale).
  * a decode sequence of length L holds L-1 cached tokens before the step;
    the step writes token L-1 (cache write) and then attends all L tokens.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np
import torch

from . import binding
from .block_manager import BLOCK_SIZE, BlockPool, SeqTable, pack_tables

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}


@dataclass
class Config:
    name: str
    title: str
    num_seqs: int                 # decode sequences
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    cache_dtype: str              # f32 | bf16 | fp8
    q_dtype: str                  # f32 | bf16
    num_blocks: int
    seed: int
    max_context: int              # table width = ceil(max_context / 16)
    lens: str                     # recipe name, see _decode_lengths
    kv_scale: float = 1.0
    partition_tokens: int = 0     # 0: library picks
    prefill_history: int = 0      # chunked-prefill request (0: none)
    prefill_chunk: int = 0
    extra: Dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def width(self) -> int:
        return -(-self.max_context // BLOCK_SIZE)


CONFIGS: Dict[str, Config] = {
    "tiny": Config(
        "tiny", "tiny paged decode, 4 seqs, shared first block (fp32)",
        num_seqs=4, num_q_heads=4, num_kv_heads=2, head_dim=64, cache_dtype="f32",
        q_dtype="f32", num_blocks=32, seed=157001, max_context=80, lens="tiny"),
    "qwen7b": Config(
        "qwen7b", "Qwen2.5-7B-shaped decode step: 64 seqs, 28/4 heads, d 128, bf16",
        num_seqs=64, num_q_heads=28, num_kv_heads=4, head_dim=128, cache_dtype="bf16",
        q_dtype="bf16", num_blocks=40000, seed=157002, max_context=4096,
        lens="uniform", extra=dict(lo=512, hi=4096)),
    "mha13b_prefix": Config(
        "mha13b_prefix", "13B-shaped MHA decode with a shared 1024-token prefix, bf16",
        num_seqs=128, num_q_heads=40, num_kv_heads=40, head_dim=128, cache_dtype="bf16",
        q_dtype="bf16", num_blocks=60000, seed=157003, max_context=4096,
        lens="lognormal_prefix", extra=dict(median=2048, sigma=1.0, lo=64, hi=4096,
                                             prefix_tokens=1024)),
    "skew_splitk": Config(
        "skew_splitk", "8 x 32768 + 248 x U[128,512] decode, 32/8 heads, bf16, 512-token partitions",
        num_seqs=256, num_q_heads=32, num_kv_heads=8, head_dim=128, cache_dtype="bf16",
        q_dtype="bf16", num_blocks=60000, seed=157004, max_context=32768,
        lens="skew", partition_tokens=512,
        extra=dict(n_long=8, long=32768, lo=128, hi=512)),
    "mixed_bf16": Config(
        "mixed_bf16", "chunked-prefill mixed step (512-row chunk over 8192 history + 96 decodes), bf16 KV",
        num_seqs=96, num_q_heads=32, num_kv_heads=8, head_dim=128, cache_dtype="bf16",
        q_dtype="bf16", num_blocks=60000, seed=157005, max_context=8704,
        lens="uniform", prefill_history=8192, prefill_chunk=512,
        extra=dict(lo=256, hi=8192)),
    "mixed_fp8": Config(
        "mixed_fp8", "chunked-prefill mixed step, fp8 e4m3 KV (scale 0.05)",
        num_seqs=96, num_q_heads=32, num_kv_heads=8, head_dim=128, cache_dtype="fp8",
        q_dtype="bf16", num_blocks=60000, seed=157005, max_context=8704,
        lens="uniform", kv_scale=0.05, prefill_history=8192, prefill_chunk=512,
        extra=dict(lo=256, hi=8192)),
}


def scaled(cfg: Config, **over) -> Config:
    """A copy of ``cfg`` with some fields replaced (smaller parity cases)."""
    d = dict(cfg.__dict__)
    d["extra"] = dict(cfg.extra)
    extra_over = over.pop("extra", None)
    d.update(over)
    if extra_over:
        d["extra"].update(extra_over)
    return Config(**d)


def _decode_lengths(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    """Context length of each decode sequence, this step's token included."""
    e = cfg.extra
    if cfg.lens == "tiny":
        return np.array(e.get("lens", [11, 7, 38, 65]), dtype=np.int64)
    if cfg.lens == "uniform":
        return rng.integers(e["lo"], e["hi"], size=cfg.num_seqs, endpoint=True)
    if cfg.lens == "lognormal_prefix":
        z = rng.standard_normal(cfg.num_seqs)
        L = np.clip(np.rint(np.exp(np.log(e["median"]) + e["sigma"] * z)), e["lo"], e["hi"])
        L = L.astype(np.int64)
        L[0::2] = np.maximum(L[0::2], e["prefix_tokens"] + 1)
        return L
    if cfg.lens == "skew":
        n_long = e["n_long"]
        short = rng.integers(e["lo"], e["hi"], size=cfg.num_seqs - n_long, endpoint=True)
        return np.concatenate([np.full(n_long, e["long"], dtype=np.int64), short])
    raise ValueError(cfg.lens)


@dataclass
class HostPlan:
    """Integer inputs of one step, all on the host."""
    cfg: Config
    context_lens: np.ndarray        # [S] int32, decode lengths incl. this step's token
    block_tables: np.ndarray        # [S, width] int32, -1 past each table's end
    slot_mapping: np.ndarray        # [T] int64 slots of this step's new tokens
    cow: List[tuple]                # (src_block, dst_block) copies to do before the write
    pool: BlockPool
    tables: List[SeqTable]
    # chunked prefill (one request), empty when the config has none
    prefill_table: Optional[np.ndarray] = None     # [1, width] int32
    prefill_context: Optional[np.ndarray] = None   # [1] int32, chunk included
    prefill_query_start: Optional[np.ndarray] = None  # [2] int32
    num_prefill_tokens: int = 0
    phase_a_lens: Optional[np.ndarray] = None      # tiny config: lengths before the step
    phase_a_tables: Optional[np.ndarray] = None


def plan_step(cfg: Config) -> HostPlan:
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    pool = BlockPool(cfg.num_blocks, seed=cfg.seed)
    slots: List[int] = []
    cow: List[tuple] = []
    pre_tab = pre_ctx = pre_qs = None
    n_pre = 0
    phase_a_lens = phase_a_tables = None

    if cfg.prefill_chunk:
        # the prefill request allocates first: history, then its chunk's slots
        req = SeqTable.allocate(pool, cfg.prefill_history)
        for _ in range(cfg.prefill_chunk):
            s, c = req.append_token()
            assert c is None
            slots.append(s)
        n_pre = cfg.prefill_chunk
        pre_tab = pack_tables([req], cfg.width)
        pre_ctx = np.array([req.num_tokens], dtype=np.int32)
        pre_qs = np.array([0, cfg.prefill_chunk], dtype=np.int32)

    lens = _decode_lengths(cfg, rng)
    tables: List[SeqTable] = []
    if cfg.lens == "tiny":
        # seqs 0 and 1 share the first block (ref_cnt 2); the block holds seq 0's
        # tokens 0-9 and seq 1 sees its first 6.  Lengths before the step are
        # lens - 1; the step's writes go through copy-on-write where needed.
        hist = lens - 1
        t0 = SeqTable.allocate(pool, int(hist[0]))
        t1 = SeqTable.with_prefix(pool, t0.blocks[:1], int(hist[1]))
        tables = [t0, t1] + [SeqTable.allocate(pool, int(h)) for h in hist[2:]]
        phase_a_lens = hist.astype(np.int32)
        phase_a_tables = pack_tables(tables, cfg.width)
    elif cfg.lens == "lognormal_prefix":
        pt = cfg.extra["prefix_tokens"] // BLOCK_SIZE
        first = None
        for i, L in enumerate(lens):
            if i % 2 == 0:
                if first is None:
                    first = SeqTable.allocate(pool, int(L) - 1)
                    tables.append(first)
                else:
                    tables.append(SeqTable.with_prefix(pool, first.blocks[:pt], int(L) - 1))
            else:
                tables.append(SeqTable.allocate(pool, int(L) - 1))
    else:
        tables = [SeqTable.allocate(pool, int(L) - 1) for L in lens]
    for t in tables:
        s, c = t.append_token()
        slots.append(s)
        if c is not None:
            cow.append(c)
    assert all(t.num_tokens == int(L) for t, L in zip(tables, lens))
    return HostPlan(cfg=cfg, context_lens=lens.astype(np.int32),
                    block_tables=pack_tables(tables, cfg.width),
                    slot_mapping=np.array(slots, dtype=np.int64), cow=cow, pool=pool,
                    tables=tables, prefill_table=pre_tab, prefill_context=pre_ctx,
                    prefill_query_start=pre_qs, num_prefill_tokens=n_pre,
                    phase_a_lens=phase_a_lens, phase_a_tables=phase_a_tables)


def _randn(shape, gen, device, chunk_elems=1 << 28):
    """N(0,1) fp32 in chunks (bounded temporaries), yielding (flat_offset, tensor)."""
    n = int(np.prod(shape))
    off = 0
    while off < n:
        m = min(chunk_elems, n - off)
        yield off, torch.randn(m, generator=gen, device=device, dtype=torch.float32)
        off += m


def _to_storage(x32: torch.Tensor, dtype: str, kv_scale: float) -> torch.Tensor:
    if dtype == "f32":
        return x32
    xb = x32.to(torch.bfloat16)
    if dtype == "bf16":
        return xb
    inv = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(kv_scale, dtype=torch.float32)
    y = (xb.float() * inv.to(x32.device)).clamp_(-448.0, 448.0)
    return y.to(torch.float8_e4m3fn)


def fill_random(t: torch.Tensor, dtype: str, gen: torch.Generator, kv_scale: float = 1.0):
    flat = t.view(-1)
    for off, x in _randn(t.shape, gen, t.device):
        flat[off:off + x.numel()] = _to_storage(x, dtype, kv_scale)
    return t


@dataclass
class Step:
    """Device tensors of one step plus its host plan."""
    plan: HostPlan
    k_cache: torch.Tensor      # [N, 16, Hkv, d]
    v_cache: torch.Tensor
    q: torch.Tensor            # [S, Hq, d] decode queries
    k_new: torch.Tensor        # [T, Hkv, d] this step's new keys (prefill chunk first)
    v_new: torch.Tensor
    slot_mapping: torch.Tensor  # [T] int64
    block_tables: torch.Tensor  # [S, width] int32
    context_lens: torch.Tensor  # [S] int32
    q_prefill: Optional[torch.Tensor] = None      # [n, Hq, d]
    prefill_table: Optional[torch.Tensor] = None
    prefill_context: Optional[torch.Tensor] = None
    prefill_query_start: Optional[torch.Tensor] = None


def make_step(cfg: Config, device="cuda", plan: Optional[HostPlan] = None) -> Step:
    """Allocate and fill every tensor of one step on ``device``."""
    plan = plan or plan_step(cfg)
    gen = torch.Generator(device=device)
    gen.manual_seed(cfg.seed)
    cdt, qdt = _TORCH_DT[cfg.cache_dtype], _TORCH_DT[cfg.q_dtype]
    shape = (cfg.num_blocks, BLOCK_SIZE, cfg.num_kv_heads, cfg.head_dim)
    k_cache = fill_random(torch.empty(shape, dtype=cdt, device=device), cfg.cache_dtype, gen,
                          cfg.kv_scale)
    v_cache = fill_random(torch.empty(shape, dtype=cdt, device=device), cfg.cache_dtype, gen,
                          cfg.kv_scale)
    S, T = cfg.num_seqs, len(plan.slot_mapping)
    q = fill_random(torch.empty((S, cfg.num_q_heads, cfg.head_dim), dtype=qdt, device=device),
                    cfg.q_dtype, gen)
    k_new = fill_random(torch.empty((T, cfg.num_kv_heads, cfg.head_dim), dtype=qdt, device=device),
                        cfg.q_dtype, gen)
    v_new = fill_random(torch.empty((T, cfg.num_kv_heads, cfg.head_dim), dtype=qdt, device=device),
                        cfg.q_dtype, gen)
    st = Step(plan=plan, k_cache=k_cache, v_cache=v_cache, q=q, k_new=k_new, v_new=v_new,
              slot_mapping=torch.from_numpy(plan.slot_mapping).to(device),
              block_tables=torch.from_numpy(plan.block_tables).to(device),
              context_lens=torch.from_numpy(plan.context_lens).to(device))
    if plan.num_prefill_tokens:
        st.q_prefill = fill_random(
            torch.empty((plan.num_prefill_tokens, cfg.num_q_heads, cfg.head_dim), dtype=qdt,
                        device=device), cfg.q_dtype, gen)
        st.prefill_table = torch.from_numpy(plan.prefill_table).to(device)
        st.prefill_context = torch.from_numpy(plan.prefill_context).to(device)
        st.prefill_query_start = torch.from_numpy(plan.prefill_query_start).to(device)
    return st


def apply_cow(step: Step) -> None:
    """Perform the plan's copy-on-write block copies on the device pools, all
    in one pa_copy_blocks launch."""
    if not step.plan.cow:
        return
    pairs = torch.tensor(step.plan.cow, dtype=torch.int64, device=step.k_cache.device)
    binding.copy_blocks(step.k_cache, step.v_cache, pairs)


def kv_bytes_per_token(cfg: Config) -> int:
    elt = {"f32": 4, "bf16": 2, "fp8": 1}[cfg.cache_dtype]
    return 2 * cfg.num_kv_heads * cfg.head_dim * elt
