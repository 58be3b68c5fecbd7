#!/usr/bin/env python3
"""Benchmark: one paged-attention step on one MI355X.

A step is the whole hot path over one batch: the cache write of the step's
new tokens (pa_reshape_and_cache), the decode attention of every sequence
(pa_decode) and, for the mixed workloads, the chunked-prefill attention
(pa_prefill_chunk).  Inputs are seeded synthetic tensors already resident in
HBM before the timed region.

    python bench.py [--steps K] [--warmup W] [--workload qwen7b] [--no-cpu-baseline]
                    [--no-configs] [--extras]
    python bench.py --workload replay_qwen7b

Prints one JSON line.  `value` is the effective KV bandwidth of the headline
step (the Qwen2.5-7B-shaped decode batch by default): KV bytes the decode
must read (each sequence's K and V rows, once) divided by the step time.

The roofline entry is for the decode launch (one kernel):
  * `achieved` / `frac`: warm, i.e. max(K, 200) back-to-back launches timed
    with one pair of HIP events on the stream the kernel runs on, right after
    the timed steps (part of a 310 MB batch then comes from the 256 MB
    Infinity Cache);
  * `cold`: the same launch with the Infinity Cache evicted before every
    launch (a 768 MiB read in between, subtracted), median and minimum, which
    is what a model's layer sees when it reads its KV once per step.
The cache write, shorter than one host submission, is timed over launches
queued behind a GPU-side wait.  As context for the 8 TB/s peak the line
also gives the box's read-stream bandwidth (the cold leg's 768 MiB reads
alone) and a plain 1 GiB device copy.  Unless --no-configs is given, the other
workloads (13B MHA with a shared prefix, the skewed long/short mix, and the
chunked-prefill mixed step with bf16 and fp8 caches) follow, each with the
same W warm-up and K timed steps, and go into `configs`.
``--extras`` adds the block copy and swap kernels and the block-size sweep.  A replay_* workload runs the continuous-batching
replay instead and reports its steady state.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

from paged_kv_cache_157_amd import binding
from paged_kv_cache_157_amd.replay import REPLAYS
from paged_kv_cache_157_amd.workload import CONFIGS, apply_cow, kv_bytes_per_token, make_step

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "paged decode attention: effective KV HBM GB/s (% of peak) and tokens/s, 1 GPU"
HOST_CORE_SHARE = 16
TIMING_LAUNCHES = 200  # least number of back-to-back launches a kernel's time is taken over


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="qwen7b", choices=sorted(CONFIGS) + sorted(REPLAYS),
                    help="a one-step workload, or a continuous-batching replay (replay_*)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="measure the headline workload only (no sub-records for the others)")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the decode with the Infinity Cache evicted")
    ap.add_argument("--extras", action="store_true",
                    help="also measure pa_copy_blocks, pa_swap_blocks and the block-size sweep "
                         "(after the timed steps)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB "
                         "(a known-size reference for hardware byte counters)")
    ap.add_argument("--traffic-json", default=os.path.join(os.path.dirname(__file__), "profiles",
                                                           "traffic.json"),
                    help="counter-measured HBM bytes per decode launch, if recorded")
    return ap.parse_args()


def algorithmic_bytes(cfg, step) -> dict:
    """Bytes the decode launch must move: K/V rows once per sequence, q, out,
    the table entries it reads and the lengths."""
    L = step.plan.context_lens.astype(np.int64)
    qb = 4 if cfg.q_dtype == "f32" else 2
    kv = int(L.sum()) * kv_bytes_per_token(cfg)
    q = cfg.num_seqs * cfg.num_q_heads * cfg.head_dim * qb
    out = cfg.num_seqs * cfg.num_q_heads * cfg.head_dim * 4
    tables = int(((L + 15) // 16).sum()) * 4 + 4 * cfg.num_seqs
    return dict(kv=kv, total=kv + q + out + tables)


def decode_kernel_name(cfg) -> str:
    """The kernel pa_decode runs for this shape: four KV heads per work-group
    when there are at least two groups of four and G >= 2, else one."""
    G = cfg.num_q_heads // cfg.num_kv_heads
    hg = cfg.num_kv_heads % 4 == 0 and cfg.num_kv_heads >= 8 and G >= 2
    return "pa::hg::decode_hg_kernel" if hg else "pa::decode_kernel"


def unique_kv_bytes(cfg, step) -> int:
    """KV bytes of the distinct physical blocks the decode reads: a block
    shared by several sequences (a common prefix) counts once, with the
    largest number of its slots any of them uses."""
    L = step.plan.context_lens.astype(np.int64)
    bt = step.plan.block_tables
    phys, fill = [], []
    for i, l in enumerate(L):
        nb = int((l + 15) // 16)
        j = np.arange(nb)
        phys.append(bt[i, :nb].astype(np.int64))
        fill.append(np.minimum(16, l - 16 * j))
    phys = np.concatenate(phys)
    fill = np.concatenate(fill)
    best = np.zeros(cfg.num_blocks, np.int64)
    np.maximum.at(best, phys, fill)
    return int(best.sum()) * kv_bytes_per_token(cfg)


def partial_bytes(cfg, step) -> int:
    """With fixed partitions: bytes of the split-K partial records, each
    (max, sum, accumulator) of G query heads written once and read once, for
    every partition of a (sequence, KV head) that has more than one."""
    pt = cfg.partition_tokens
    if pt <= 0:
        return 0
    parts = (step.plan.context_lens.astype(np.int64) + pt - 1) // pt
    G = cfg.num_q_heads // cfg.num_kv_heads
    return int(parts[parts > 1].sum()) * cfg.num_kv_heads * G * (cfg.head_dim + 2) * 4 * 2


def host_cpus() -> dict:
    """The host's logical CPUs and the ones this process may run on."""
    try:
        allowed = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        allowed = os.cpu_count() or 1
    return dict(host_logical_cpus=os.cpu_count() or 1, allowed_cpus=allowed)


def cpu_baseline(cfg, step) -> dict:
    """The CPU oracle, as it stands, on a bounded sample of the same batch.
    It runs with one thread per CPU this process may use, at most the box's
    16-CPU share of the host (OMP_NUM_THREADS when set)."""
    import oracle  # test infrastructure: used only for this baseline leg

    def host_bits(t):
        if t.dtype == torch.float32:
            return t.cpu().numpy()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.view(torch.uint8).cpu().numpy()

    def pool_rows(a):
        return a.reshape(a.shape[0] * a.shape[1], a.shape[2], a.shape[3])

    cpus = host_cpus()
    share = int(os.environ.get("OMP_NUM_THREADS", HOST_CORE_SHARE) or HOST_CORE_SHARE)
    cores = max(1, min(share, cpus["allowed_cpus"]))
    kp = host_bits(step.k_cache)
    vp = host_bits(step.v_cache)
    q = host_bits(step.q)
    L = step.plan.context_lens
    order = np.argsort(-L)  # a deterministic sample: sequences in length order
    # whole passes over the batch until about 10 s have been spent (a long
    # batch stops inside its first pass after 15 s)
    min_s, budget_s, used = 10.0, 15.0, 0.0
    done_bytes = 0
    n_seq = 0
    t0 = time.time()
    while used < min_s:
        for i in order:
            sel_seq = np.full(cfg.num_q_heads, i, np.int32)
            sel_head = np.arange(cfg.num_q_heads, dtype=np.int32)
            oracle.decode(q, pool_rows(kp), pool_rows(vp), step.plan.block_tables, L, cfg.scale,
                          kv_scale=cfg.kv_scale, sel_seq=sel_seq, sel_head=sel_head,
                          num_threads=cores)
            done_bytes += int(L[i]) * kv_bytes_per_token(cfg)
            n_seq += 1
            used = time.time() - t0
            if used > budget_s:
                break
        if used > budget_s:
            break
    passes = n_seq / cfg.num_seqs
    return dict(value=round(done_bytes / used / 1e9, 4), unit="GB/s", cores=cores, kind="oracle",
                sample=f"{n_seq} sequence decodes ({passes:.2f} passes over the {cfg.num_seqs}-sequence "
                       f"batch, longest first), all {cfg.num_q_heads} heads, {used:.1f} s",
                **cpus)


class Timer:
    """GPU-side timing helpers on torch's current stream (the stream every
    libpa call of this script is queued on)."""

    def __init__(self):
        self.e0 = torch.cuda.Event(enable_timing=True)
        self.e1 = torch.cuda.Event(enable_timing=True)
        # torch.cuda._sleep spins for a number of GPU clock ticks; ticks per
        # millisecond are measured once here
        probe_ticks = 1 << 22
        torch.cuda._sleep(probe_ticks)
        self.e0.record()
        torch.cuda._sleep(probe_ticks)
        self.e1.record()
        torch.cuda.synchronize()
        self.ticks_per_ms = probe_ticks / max(self.e0.elapsed_time(self.e1), 1e-3)

    def launch_ms(self, fn, n, hold=False):
        """Average duration of one launch of fn: HIP events recorded on the stream
        the kernels run on (torch's current stream) around n back-to-back launches
        (one event pair, so the event cost is spread over n launches).  With
        `hold`, the launches are queued behind a GPU-side wait long enough for
        the host to submit all of them, so that a kernel shorter than one host
        submission (the cache write) is timed on the GPU and not at the host's
        pace.  Longer kernels are timed without it: the GPU is then the
        bottleneck anyway, and an idle wait lets its clocks drop."""
        fn()
        if hold:
            torch.cuda._sleep(int(self.ticks_per_ms * (0.5 + 0.03 * n)))
        self.e0.record()
        for _ in range(n):
            fn()
        self.e1.record()
        torch.cuda.synchronize()
        return self.e0.elapsed_time(self.e1) / n

    def cold_us(self, fn, evict, n=20, reps=5):
        """Launch time of fn with its inputs evicted from the 256 MB Infinity
        Cache: n rounds of (a read of `evict`, larger than that cache, then fn)
        back to back, minus n reads alone, per round; median and minimum over
        `reps` repetitions.  The reads alone also give the box's read-stream
        bandwidth (median over the repetitions)."""
        ts, rd = [], []
        for _ in range(reps):
            t = []
            for with_fn in (True, False):
                evict.sum()
                torch.cuda.synchronize()
                self.e0.record()
                for _ in range(n):
                    evict.sum()
                    if with_fn:
                        fn()
                self.e1.record()
                torch.cuda.synchronize()
                t.append(self.e0.elapsed_time(self.e1))
            ts.append((t[0] - t[1]) / n * 1e3)
            rd.append(n * evict.numel() * evict.element_size() / (t[1] * 1e-3) / 1e9)
        return dict(median_us=round(float(np.median(ts)), 2), min_us=round(float(np.min(ts)), 2),
                    launches=n * reps, read_stream_gbs=round(float(np.median(rd)), 1))


def prefill_flops(cfg) -> int:
    """4 d Hq flops (QK^T and PV) per (query row, attended key) of the chunk:
    row j of the chunk attends history + j + 1 keys."""
    return cfg.num_q_heads * cfg.head_dim * 4 * sum(
        cfg.prefill_history + j + 1 for j in range(cfg.prefill_chunk))


def measure(cfg, args, dev, timer: Timer, headline: bool) -> dict:
    """One workload: W warm-up and K timed steps (cache write, [prefill,]
    decode) back to back, then the per-launch times of its kernels."""
    print(f"bench: {cfg.name}: inputs", file=sys.stderr, flush=True)
    step = make_step(cfg, dev)
    out = torch.empty(step.q.shape, dtype=torch.float32, device=dev)
    out_pre = None
    if step.q_prefill is not None:
        out_pre = torch.empty(step.q_prefill.shape, dtype=torch.float32, device=dev)
    apply_cow(step)
    torch.cuda.synchronize()

    def cache_write():
        binding.reshape_and_cache(step.k_new, step.v_new, step.k_cache, step.v_cache,
                                  step.slot_mapping, kv_scale=cfg.kv_scale)

    def prefill():
        binding.prefill_chunk(out_pre, step.q_prefill, step.k_cache, step.v_cache,
                              step.prefill_table, step.prefill_query_start, step.prefill_context,
                              cfg.scale, kv_scale=cfg.kv_scale)

    def decode():
        binding.decode(out, step.q, step.k_cache, step.v_cache, step.block_tables,
                       step.context_lens, cfg.scale, partition_tokens=cfg.partition_tokens,
                       kv_scale=cfg.kv_scale)

    def run_step():
        cache_write()
        if out_pre is not None:
            prefill()
        decode()

    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()

    # the timed region: K whole steps back to back (no events inside: an event
    # record costs several microseconds of GPU idle time on this stack)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    print(f"bench: {cfg.name}: {args.steps} steps in {ms_per_step * args.steps:.1f} ms",
          file=sys.stderr, flush=True)
    # per-launch times: at least TIMING_LAUNCHES back-to-back launches, so that
    # a short run (few timed steps) does not report its first, slow launches
    n_time = max(args.steps, TIMING_LAUNCHES)
    dec_ms = timer.launch_ms(decode, n_time)
    pre_ms = timer.launch_ms(prefill, n_time) if out_pre is not None else None
    # held launches: at most 200 per event pair (HIP's queue depth)
    cw_ms = timer.launch_ms(cache_write, min(args.steps, 200), hold=True)

    ab = algorithmic_bytes(cfg, step)
    uniq = unique_kv_bytes(cfg, step)
    tokens_per_step = cfg.num_seqs + (cfg.prefill_chunk if out_pre is not None else 0)
    kv_gbs = ab["kv"] / (ms_per_step * 1e-3) / 1e9
    rec = dict(
        workload=f"{cfg.name}: {cfg.title}",
        num_seqs=cfg.num_seqs, q_heads=cfg.num_q_heads, kv_heads=cfg.num_kv_heads,
        head_dim=cfg.head_dim, cache_dtype=cfg.cache_dtype, block_size=16,
        pool_blocks=cfg.num_blocks, partition_tokens=cfg.partition_tokens,
        context_tokens=int(step.plan.context_lens.sum()),
        new_tokens=int(len(step.plan.slot_mapping)), seed=cfg.seed,
        steps=args.steps, warmup=args.warmup,
        ms_per_step=round(ms_per_step, 5),
        step_kv_gbs=round(kv_gbs, 2),
        tokens_per_step=tokens_per_step,
        tokens_per_s=round(tokens_per_step / (ms_per_step * 1e-3), 1),
        decode_kernel=decode_kernel_name(cfg),
        decode_us=round(dec_ms * 1e3, 2),
        decode_kv_bytes=ab["kv"],
        decode_algorithmic_bytes=ab["total"],
        decode_kv_gbs=round(ab["kv"] / (dec_ms * 1e-3) / 1e9, 2),
        decode_achieved_gbs=round(ab["total"] / (dec_ms * 1e-3) / 1e9, 2),
        decode_frac_of_hbm_peak=round(ab["total"] / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        cache_write_us=round(cw_ms * 1e3, 2),
    )
    if uniq < ab["kv"]:  # shared blocks: the distinct bytes read as well
        rec["unique_kv_bytes"] = uniq
        rec["decode_unique_kv_gbs"] = round(uniq / (dec_ms * 1e-3) / 1e9, 2)
    if cfg.partition_tokens > 0:
        rec["partial_bytes_per_launch"] = partial_bytes(cfg, step)
    if pre_ms is not None:
        fl = prefill_flops(cfg)
        rec["prefill_us"] = round(pre_ms * 1e3, 2)
        rec["prefill_gflop"] = round(fl / 1e9, 2)
        rec["prefill_tflops"] = round(fl / (pre_ms * 1e-3) / 1e12, 2)
        rec["prefill_pct_of_bf16_mfma_peak"] = round(
            100.0 * rec["prefill_tflops"] / MFMA_BF16_PEAK_TFLOPS, 2)
    if headline and not args.no_cold:
        evict = torch.ones(192 << 20, dtype=torch.float32, device=dev)  # 768 MiB
        cold = timer.cold_us(decode, evict)
        del evict
        cold["achieved_gbs"] = round(ab["total"] / (cold["median_us"] * 1e-6) / 1e9, 2)
        cold["frac"] = round(cold["achieved_gbs"] / HBM_PEAK_GBS, 4)
        rec["decode_cold"] = cold
    if headline:
        rec["_step"] = step
        rec["_fns"] = dict(decode=decode, cache_write=cache_write, out=out)
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    binding.load()
    if args.workload in REPLAYS:
        replay_main(args)
        return
    cfg = CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    timer = Timer()
    head = measure(cfg, args, dev, timer, headline=True)
    step = head.pop("_step")
    fns = head.pop("_fns")
    decode, out = fns["decode"], fns["out"]
    launch_ms = timer.launch_ms

    # copy-on-write copies (pa_copy_blocks): up to 1024 pairs from blocks the
    # batch uses into free blocks, so no table's data changes
    free = step.plan.pool.free_blocks()[:1024] if args.extras else []
    used = np.unique(step.plan.block_tables[step.plan.block_tables >= 0])
    copy_res = None
    if free and len(used):
        rng = np.random.default_rng(cfg.seed)
        pairs = np.stack([rng.choice(used, len(free)), np.array(free)], 1).astype(np.int64)
        pairs_d = torch.from_numpy(pairs).to(dev)
        blk = kv_bytes_per_token(cfg) // 2 * 16  # one block of one pool
        cp_ms = launch_ms(lambda: binding.copy_blocks(step.k_cache, step.v_cache, pairs_d),
                          min(args.steps, 200), hold=True)
        moved = 2 * 2 * len(free) * blk  # both pools, read and write
        copy_res = dict(pairs=len(free), us=round(cp_ms * 1e3, 2),
                        gbs=round(moved / (cp_ms * 1e-3) / 1e9, 1))

    # swapping (pa_swap_blocks): up to 1024 of the batch's blocks out to pinned
    # host pools and back into free device blocks, against a contiguous copy
    # of the same bytes over the host link and the pages' cost model
    swap_res = None
    if free and len(used):
        from paged_kv_cache_157_amd.block_manager import swap_time_model

        n = len(free)
        hshape = (n,) + tuple(step.k_cache.shape[1:])
        hk = torch.empty(hshape, dtype=step.k_cache.dtype).pin_memory()
        hv = torch.empty(hshape, dtype=step.k_cache.dtype).pin_memory()
        outp = torch.from_numpy(np.stack([used[:n], np.arange(n)], 1).astype(np.int64)).to(dev)
        inp = torch.from_numpy(np.stack([np.arange(n), np.array(free)], 1).astype(np.int64)).to(dev)
        out_ms = launch_ms(lambda: binding.swap_blocks(step.k_cache, step.v_cache, hk, hv, outp), 20)
        in_ms = launch_ms(lambda: binding.swap_blocks(hk, hv, step.k_cache, step.v_cache, inp), 20)
        nbytes = 2 * n * (kv_bytes_per_token(cfg) // 2 * 16)
        flat_d = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        flat_h = torch.empty(nbytes, dtype=torch.uint8).pin_memory()
        d2h_ms = launch_ms(lambda: flat_h.copy_(flat_d, non_blocking=True), 20)
        h2d_ms = launch_ms(lambda: flat_d.copy_(flat_h, non_blocking=True), 20)
        link = nbytes / (0.5 * (d2h_ms + h2d_ms) * 1e-3)
        swap_res = dict(blocks=n, bytes=nbytes, out_us=round(out_ms * 1e3, 1),
                        in_us=round(in_ms * 1e3, 1),
                        out_gbs=round(nbytes / (out_ms * 1e-3) / 1e9, 1),
                        in_gbs=round(nbytes / (in_ms * 1e-3) / 1e9, 1),
                        d2h_copy_gbs=round(nbytes / (d2h_ms * 1e-3) / 1e9, 1),
                        h2d_copy_gbs=round(nbytes / (h2d_ms * 1e-3) / 1e9, 1),
                        round_trip_model_us=round(
                            swap_time_model(n * 16, kv_bytes_per_token(cfg), link) * 1e6, 1))
        del hk, hv, flat_d, flat_h

    # block-size trade-off ([L33] §2.2, appendix Q3): the batch's lengths
    # decoded from pools of 8-, 16-, 32- and 64-token blocks, scattered at random
    bs_res = None
    if args.extras and cfg.cache_dtype == "bf16":
        bs_res = {}
        L = step.plan.context_lens.astype(np.int64)
        for B in (8, 16, 32, 64):
            nbs = (L + B - 1) // B
            nblk = int(nbs.sum()) + 64
            rng = np.random.default_rng(cfg.seed + B)
            perm = rng.permutation(nblk)
            bt = np.full((len(L), int(nbs.max())), -1, np.int32)
            c = 0
            for i, n in enumerate(nbs):
                bt[i, :n] = perm[c:c + n]
                c += n
            shp = (nblk, B, cfg.num_kv_heads, cfg.head_dim)
            kb = torch.randn(shp, device=dev).to(torch.bfloat16)
            vb = torch.randn(shp, device=dev).to(torch.bfloat16)
            bt_d = torch.from_numpy(bt).to(dev)
            run = lambda: binding.decode(out, step.q, kb, vb, bt_d, step.context_lens, cfg.scale)
            for _ in range(50):
                run()
            us = launch_ms(run, 300) * 1e3
            bs_res[str(B)] = dict(decode_us=round(us, 2), table_entries=int(nbs.sum()),
                                  tail_waste_tokens=int((nbs * B - L).sum()))
            del kb, vb

    # bandwidth context: a plain 1 GiB device copy (reads and writes 1 GiB)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    timer.e0.record()
    for _ in range(5):
        dst.copy_(src)
    timer.e1.record()
    torch.cuda.synchronize()
    copy_gbs = round(2 * (1 << 30) * 5 / (timer.e0.elapsed_time(timer.e1) * 1e-3) / 1e9, 1)
    del src, dst
    if args.copy_probe_mib:
        # a plain device copy of known size: rocprofv3 --pmc reads of FETCH_SIZE /
        # WRITE_SIZE for it convert the counters into bytes
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    traffic = None
    if os.path.exists(args.traffic_json):
        from paged_kv_cache_157_amd.rocprof_summary import decode_source_hash
        try:
            rec = json.load(open(args.traffic_json)).get(cfg.name)
            if rec and rec.get("source_hash") == decode_source_hash():
                traffic = rec.get("bytes_per_launch")  # counters of this very kernel
        except (OSError, ValueError):
            traffic = None

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, step)
    del step, out, decode, fns
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    # the other workloads, one after another (each freed before the next)
    subs = {}
    if not args.no_configs:
        for name in ("mha13b_prefix", "skew_splitk", "mixed_bf16", "mixed_fp8"):
            if name == cfg.name:
                continue
            subs[name] = measure(CONFIGS[name], args, dev, timer, headline=False)
            torch.cuda.synchronize()
            torch.cuda.empty_cache()

    dec_us = head["decode_us"]
    cold = head.get("decode_cold")
    read_gbs = cold.pop("read_stream_gbs", None) if cold else None
    res = {
        "metric": METRIC,
        "value": head["step_kv_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.cache_dtype,
        "data": "synthetic",
        "config": {"workload": head["workload"], "num_seqs": cfg.num_seqs,
                   "q_heads": cfg.num_q_heads, "kv_heads": cfg.num_kv_heads,
                   "head_dim": cfg.head_dim, "block_size": 16, "pool_blocks": cfg.num_blocks,
                   "context_tokens": head["context_tokens"], "new_tokens": head["new_tokens"],
                   "seed": cfg.seed},
        "pct_of_hbm_peak": round(100.0 * head["step_kv_gbs"] / HBM_PEAK_GBS, 2),
        "tokens_per_step": head["tokens_per_step"],
        "tokens_per_s": head["tokens_per_s"],
        "decode_us": dec_us,
        "decode_kv_gbs": head["decode_kv_gbs"],
        "cache_write_us": head["cache_write_us"],
        "roofline": {"bound": "hbm", "achieved": head["decode_achieved_gbs"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": head["decode_frac_of_hbm_peak"],
                     "traffic": traffic,
                     "kernel": f"pa_decode ({head['decode_kernel']}, one launch)",
                     "algorithmic_bytes_per_launch": head["decode_algorithmic_bytes"],
                     "timing": f"warm: {max(args.steps, TIMING_LAUNCHES)} back-to-back launches "
                               f"after the timed steps, one HIP event pair, {dec_us} us per launch",
                     "cold": None if cold is None else dict(
                         cold, timing="Infinity Cache evicted before every launch (768 MiB read, "
                                      "subtracted); median and minimum over 5 x 20 launches")},
        "device_copy_gbs": copy_gbs,
        "read_stream_gbs": read_gbs,
        "copy_blocks": copy_res,
        "swap_blocks": swap_res,
        "block_size_sweep": bs_res,
    }
    for k in ("unique_kv_bytes", "decode_unique_kv_gbs", "partial_bytes_per_launch", "prefill_us",
              "prefill_tflops", "prefill_pct_of_bf16_mfma_peak"):
        if k in head:
            res[k] = head[k]
    if subs:
        res["configs"] = subs
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


def replay_main(args):
    """A continuous-batching replay: every step schedules decodes and prefill
    chunks under the token budget and runs the copy, cache-write, prefill and
    decode kernels; the line reports the steady state in GPU time (HIP events
    around each step's kernels) and the wall time including host scheduling."""
    from paged_kv_cache_157_amd import replay

    cfg = REPLAYS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    replay.run(cfg, dev, max_steps=min(args.warmup, 50))  # warms up the kernels and the allocator
    r = replay.run(cfg, dev)
    print(json.dumps({
        "metric": "continuous-batching replay: tokens/s and decode KV GB/s in GPU time, 1 GPU",
        "value": r["tokens_per_s_gpu"], "unit": "tokens/s", "n_gpus": 1,
        "steps": r["steps"], "warmup": min(args.warmup, 50),
        "ms_per_step": r["gpu_ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.cache_dtype, "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.num_requests} requests, prompts U{list(cfg.prompt)}, "
                               f"outputs U{list(cfg.output)}, budget {cfg.budget} tokens/step",
                   "q_heads": cfg.num_q_heads, "kv_heads": cfg.num_kv_heads,
                   "head_dim": cfg.head_dim, "pool_blocks": cfg.num_blocks, "seed": cfg.seed},
        "replay": r}), flush=True)


if __name__ == "__main__":
    main()
