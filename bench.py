"""Benchmark: paged decode attention on one MI355X.

One step = the whole decode hot path over one batch: copy-on-write block
copies (if the step has any), pa_write_kv of every sequence's new token, and
pa_decode over the batch.  The default workload is the Llama-3.1-8B-like GQA
layer (32 query / 8 KV heads, head_dim 128, bf16 cache, B = 16, 256
sequences in groups of 8 sharing a 1008-token prefix, lognormal private
lengths).  Inputs are resident in HBM before timing starts; steps rotate over
several copies of the cache so no step finds the previous step's data in the
caches.

Prints ONE JSON line (rank 0, N = 1): value = logical KV bytes read per step
/ step time (GB/s).  Before its W warmup steps each decode measurement runs
untimed steps until the GPU's clocks have settled (``prewarm_steps``: at
least 100 steps and 50 ms), so a short timed run reads the steady state.
The K timed steps run with nothing else on the stream; ``roofline`` is then
measured live with HIP events around every pa_decode call of K more steps
(partition + combine launches; event records would add ~6.5 us to each
step of the timed region, so they are kept out of it);
beside its algorithmic ``frac`` it carries ``hbm_frac`` (the call's HBM bytes
from the committed rocprofv3 counter summary, over the same time) and the
rate of unique KV bytes.  ``cpu_baseline`` times the float64 oracle on every
available host core.

Nested objects in the same line:
  noshare      the same step with every prefix private (logical = unique
               bytes), with its own roofline and oracle baseline;
  block_sweep  B = 8 / 16 / 32 at ctx 1000 x 128: paged, contiguous-layout
               and identity-placement pa_decode times and the overheads;
  ceiling      plain streaming read and scattered 4 KiB-tile read rates,
               with the default and the non-temporal cache policy;
  prefill      pa_prefill on the Llama-3.1-8B-like prefill batch, TFLOP/s
               against the dense bf16 matrix-core peak;
  prefix_cache, swap, fp8   the prefix cache, the preemption copies, and the
               decode step over an E4M3 copy of the cache;
  configs      the Llama-7B-like MHA step, the LLaMA-13B-like layer at
               context 4096 and its 4-beam copy-on-write batch.
``--mode decode|prefill|prefix|swap|fp8|ceiling`` prints one alone.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--mode ...] [--no-extras]
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention: KV HBM GB/s (% of MI355X peak); sequences/sec"
PEAK_HBM_GBPS = 8000.0
# Untimed decode steps before the warmup steps (clock settling): at least this many, and
# at least this long.
PREWARM_STEPS = 100
PREWARM_S = 0.05
PREFILL_METRIC = "paged prefill attention: algorithmic TFLOP/s (% of MI355X dense bf16 matrix-core peak)"
PEAK_MFMA_BF16_TFLOPS = 2500.0
WORKLOADS = {
    "llama31_8b_gqa": ("gqa", "Llama-3.1-8B-like GQA decode layer, shared 1008-token prefixes"),
    "llama31_8b_gqa_noshare": ("gqa_noshare", "same lengths and bytes, every prefix private"),
    "llama7b_mha": ("llama7b", "Llama-7B-like MHA decode layer"),
    "sweep_b8": ("sweep8", "ctx 1000 x 128, B=8"),
    "sweep_b16": ("sweep16", "ctx 1000 x 128, B=16"),
    "sweep_b32": ("sweep32", "ctx 1000 x 128, B=32"),
    "llama13b_long": ("long13b", "LLaMA-13B-like MHA layer, ctx 4096 x 32"),
    "llama13b_beam": ("beam13b", "8 parents x 4 beams at ctx 4096, copy-on-write"),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pa_decode_traffic.md")
PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pa_prefill_traffic.md")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def elem_bytes(dtype):
    return {"f32": 4, "f16": 2, "bf16": 2}[dtype]


def decode_bytes(wl, ctx):
    """Algorithmic bytes of one pa_decode launch: every KV row of every context
    once, q, the float32 output, the table entries read and the lengths."""
    e = elem_bytes(wl.dtype)
    S, Hq, Hkv, d, B = wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size
    kv = int(sum(ctx)) * 2 * Hkv * d * e
    other = S * Hq * d * e + S * Hq * d * 4 + sum(4 * ((c + B - 1) // B) for c in ctx) + 4 * S
    return kv, kv + other


def source_digest(names=("decode.hip", "decode_params.h", "device_common.h")):
    """Digest of the kernel sources' code: comments, indentation and blank
    lines are left out, so a comment edit does not retire a counter summary."""
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "paged_kv_cache_147_amd", "csrc", name), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(line.strip() for line in text.splitlines() if line.strip())
        h.update(code.encode("utf-8"))
    return h.hexdigest()[:16]


def measured_prefill_traffic():
    """Per-launch HBM bytes of pa_prefill from the committed counter summary,
    or None when the prefill source changed since the counters were taken."""
    try:
        text = open(PREFILL_TRAFFIC_FILE, encoding="utf-8").read()
    except OSError:
        return None
    m = re.search(r"^\|\s*llama31_8b_prefill\s*\|\s*([0-9a-f]{16})\s*\|\s*([0-9.e+]+)\s*\|", text, flags=re.M)
    if not m or m.group(1) != source_digest(("prefill.hip", "device_common.h")):
        return None
    return float(m.group(2))


def measured_traffic(workload):
    """Per-launch HBM bytes from the committed counter summary, or None when
    the decode kernel source changed since the counters were taken."""
    try:
        text = open(TRAFFIC_FILE, encoding="utf-8").read()
    except OSError:
        return None
    m = re.search(r"^\|\s*" + re.escape(workload) + r"\s*\|\s*([0-9a-f]{16})\s*\|\s*([0-9.e+]+)\s*\|",
                  text, flags=re.M)
    if not m or m.group(1) != source_digest():
        return None
    return float(m.group(2))


def host_cpu():
    """The host's CPU model (from /proc/cpuinfo) and the cores this process may use."""
    model = None
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = os.cpu_count()
    return {"cpu_model": model, "cores_available": avail}


# ---- CPU baselines --------------------------------------------------------------
# The oracle runs in processes forked from this one, one per available core,
# before anything initialises the GPU (a process that holds the GPU is never
# forked).  Each process sees the parent's arrays copy-on-write, runs with one
# BLAS thread, and works on its own share of the sequences.

_FORK = {}


def _one_thread():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _noop(_):
    return None


def fork_map(worker, chunks, min_wall=2.0, max_reps=16):
    """Runs worker(chunk) over all chunks on one forked process per available
    core; repeats the whole map until ~min_wall seconds.  Returns (wall time
    of one map, cores used, repetitions)."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    cores = host_cpu()["cores_available"]
    with ProcessPoolExecutor(max_workers=cores, mp_context=mp.get_context("fork"), initializer=_one_thread) as ex:
        list(ex.map(_noop, range(4 * cores)))          # every worker started before timing
        walls = []
        while not walls or (sum(walls) < min_wall and len(walls) < max_reps):
            t0 = time.perf_counter()
            list(ex.map(worker, chunks))
            walls.append(time.perf_counter() - t0)
    return min(walls), cores, len(walls)


def _chunks(n, parts):
    step = max(1, -(-n // parts))
    return [slice(a, min(n, a + step)) for a in range(0, n, step)]


def _decode_chunk(sl):
    from oracle import attention as A
    st = _FORK["decode"]
    A.paged_decode(st["q"][sl], st["k"], st["v"], st["tables"][sl], st["lens"][sl], st["B"], st["scale"],
                   st["dtype"], st["Hq"], st["Hkv"])


def cpu_baseline(wl):
    """The float64 oracle, as it stands, over the whole batch on every
    available core; GB/s of logical KV."""
    import numpy as np

    from tests._replay import OracleRun
    run = OracleRun(wl)
    tables, lens = run.tables(wl)
    _FORK["decode"] = dict(q=wl.q, k=run.cache.k, v=run.cache.v, tables=tables, lens=lens, B=wl.block_size,
                           scale=wl.scale, dtype=wl.dtype, Hq=wl.num_q_heads, Hkv=wl.num_kv_heads)
    # longest sequences first, in small chunks, so the processes finish together
    order = np.argsort(-lens, kind="stable")
    _FORK["decode"].update(q=wl.q[order], tables=tables[order], lens=lens[order])
    cores = host_cpu()["cores_available"]
    wall, cores, reps = fork_map(_decode_chunk, _chunks(wl.num_seqs, 8 * cores))
    kv = int(np.sum(lens)) * 2 * wl.num_kv_heads * wl.head_dim * elem_bytes(wl.dtype)
    del _FORK["decode"]
    return {"value": round(kv / wall / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"all {wl.num_seqs} sequences ({kv / 1e9:.3f} GB logical KV) on {cores} forked processes, "
                      f"{wall:.2f} s wall (best of {reps}), float64 numpy",
            "seqs_per_s": round(wl.num_seqs / wall, 2), **host_cpu()}


def prefill_flops(ctx, q_start, head_dim, num_q_heads):
    """Algorithmic flops of one pa_prefill launch: a chunk row at position p
    takes p + 1 dot products of length d (scores) and p + 1 d-wide
    multiply-adds (p.V), 2 flops per multiply-add, for every query head.
    Rows of a chunk of n sit at positions ctx - n .. ctx - 1."""
    total = 0
    for s in range(len(ctx)):
        n = int(q_start[s + 1]) - int(q_start[s])
        first = int(ctx[s]) - n
        total += n * first + n * (n + 1) // 2
    return total * 4 * head_dim * num_q_heads


def _prefill_chunk(job):
    from oracle import prefill as PF
    st = _FORK["prefill"]
    s, r0, r1 = job
    rows = [(r, h) for r in range(r0, r1) for h in range(st["Hq"])]
    PF.paged_prefill(st["q_rows"], st["k"], st["v"], st["tables"], st["lens"], st["qs"], st["B"], st["scale"],
                     st["dtype"], st["Hq"], st["Hkv"], rows=rows)


def prefill_cpu_baseline(wl):
    """The float64 prefill oracle, as it stands, over the whole batch (every
    chunk row and head) on every available core; TFLOP/s."""
    from tests._replay import OracleRun
    run = OracleRun(wl)
    tables, lens = run.tables(wl)
    qs = [int(x) for x in wl.info["q_start"]]
    _FORK["prefill"] = dict(q_rows=wl.info["q_rows"], k=run.cache.k, v=run.cache.v, tables=tables, lens=lens,
                            qs=qs, B=wl.block_size, scale=wl.scale, dtype=wl.dtype, Hq=wl.num_q_heads,
                            Hkv=wl.num_kv_heads)
    jobs = []
    for s in range(wl.num_seqs):                 # 32-row jobs
        jobs += [(s, r, min(r + 32, qs[s + 1])) for r in range(qs[s], qs[s + 1], 32)]
    jobs = jobs[::4]                             # a bounded sample: every fourth job, every head
    jobs.sort(key=lambda j: -int(lens[j[0]]))    # longest contexts first
    wall, cores, reps = fork_map(_prefill_chunk, jobs, min_wall=1.0, max_reps=2)
    del _FORK["prefill"]
    d, Hq = wl.head_dim, wl.num_q_heads
    # a chunk row at position p costs (p + 1) dot products and (p + 1) multiply-adds of d, per head
    flops = sum(4 * d * Hq * (int(lens[s]) - (qs[s + 1] - qs[s]) + (r - qs[s]) + 1)
                for s, r0, r1 in jobs for r in range(r0, r1))
    return {"value": round(flops / wall / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"every fourth 32-row job of the {wl.num_seqs}-sequence batch, every head "
                      f"({flops / 1e9:.1f} GFLOP) on {cores} forked processes, {wall:.2f} s wall (best of {reps}), "
                      f"float64 numpy", **host_cpu()}


def bench_prefill(wl, steps, warmup, dev, cpu=None):
    """pa_prefill on the Llama-3.1-8B-like prefill batch: `steps` launches
    timed by the host clock, then `steps` more each between HIP events on the
    stream it runs on (timed_passes)."""
    import numpy as np
    import torch

    import paged_kv_cache_147_amd as P
    import workloads as W
    from tests._native import NativeDeviceRun, device_tensor
    run = NativeDeviceRun(wl, device=dev)
    ctx = run.ctx_host.tolist()
    qs = [int(x) for x in wl.info["q_start"]]
    q = device_tensor(wl.info["q_rows"], wl.dtype, dev)
    q_start = torch.tensor(qs, dtype=torch.int32, device=dev)
    max_chunk = int(max(wl.info["chunk"]))
    out = torch.empty((q.shape[0], wl.num_q_heads, wl.head_dim), dtype=torch.float32, device=dev)
    stream = P.current_stream(dev)
    flops = prefill_flops(ctx, qs, wl.head_dim, wl.num_q_heads)

    def call(i=0, ev=None):
        if ev is not None:
            ev[0].record()
        P.pa_prefill(out, q, run.k_cache, run.v_cache, run.tables, run.ctx, q_start, wl.scale, max_chunk,
                     stream=stream)
        if ev is not None:
            ev[1].record()

    for _ in range(warmup):
        call()
    ms_call, ms = timed_passes(call, 0, steps)
    avg = float(np.mean(ms))
    log(f"[bench] prefill: {steps} launches, {ms_call:.4f} ms/call wall; kernel avg {avg:.4f} ms "
        f"(p10 {np.percentile(ms, 10):.4f}, p90 {np.percentile(ms, 90):.4f})")
    tflops = flops / (ms_call * 1e-3) / 1e12
    achieved = flops / (avg * 1e-3) / 1e12
    res = {
        "metric": PREFILL_METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_call, 5),
        "higher_is_better": True,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama31_8b_prefill",
                   "description": "Llama-3.1-8B-like GQA layer, 16 sequences, 512-token chunks after "
                                  "cached prefixes of 0..2048 tokens",
                   "batch": wl.num_seqs, "chunk_rows": qs[-1], "num_q_heads": wl.num_q_heads,
                   "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim, "block_size": wl.block_size,
                   "kv_dtype": wl.dtype, "out_dtype": "f32", "ctx_mean": round(float(np.mean(ctx)), 1),
                   "ctx_max": int(max(ctx)), "flops_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_MFMA_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_MFMA_BF16_TFLOPS, 4),
                     "traffic": measured_prefill_traffic(), "kernel": "pa_prefill (one launch)",
                     "avg_launch_ms": round(avg, 5), "flops_per_launch": flops,
                     "launch_ms_p10_median_p90": [round(float(np.percentile(ms, x)), 5) for x in (10, 50, 90)]},
        "cpu_baseline": cpu,
    }
    return res


def bench_prefix(dev, with_cpu, rounds=200, reps=20):
    """Prefix cache on a batch of 16 requests that share a 1024-token system
    prompt, each with a private 512-token question (Llama-3.1-8B-like GQA
    layer, bf16, B = 16).
    Host: admissions per second through pa_seq_alloc_prefix (each round
    admits and releases all 16; from the second request on, the system
    prompt's 64 blocks are found in the cache).
    GPU: pa_prefill of the batch with the system prompt recomputed (1536-row
    chunks) and with it cached (512-row chunks over the same 1536-token
    contexts, through the shared blocks), HIP events around each launch.
    The oracle model's admissions per second are the CPU baseline."""
    import numpy as np
    import torch

    import paged_kv_cache_147_amd as P
    S, SYS, Q, B, Hq, Hkv, D = 16, 1024, 512, 16, 32, 8, 128
    rng = np.random.default_rng(0)
    system = rng.integers(0, 128000, size=SYS)
    # every admission brings a question of its own; only the system prompt repeats
    prompts = [[np.concatenate([system, rng.integers(0, 128000, size=Q)]).astype(np.int32) for _ in range(S)]
               for _ in range(rounds + 2)]
    nblocks = S * (SYS + Q) // B + 64
    pool = P.BlockPool(nblocks, B)
    pool.enable_prefix_cache()

    def admit_all(p, base, r):
        return [p.alloc_prefix(base + s, prompts[r][s], salt=7)[0] for s in range(S)]

    admit_all(pool, 0, 0)                  # warm: the system prompt is now cached
    for s in range(S):
        pool.free(s)
    t0 = time.perf_counter()
    for r in range(rounds):
        admit_all(pool, (r + 1) * S, r + 1)
        for s in range(S):
            pool.free((r + 1) * S + s)
    host_s = time.perf_counter() - t0
    st = pool.prefix_stats()
    cached = admit_all(pool, 10 ** 6, rounds + 1)   # the batch the GPU runs
    tables, ctx = pool.block_tables([10 ** 6 + s for s in range(S)], (SYS + Q) // B)
    shared = int(np.sum(tables[:, :SYS // B] == tables[0, :SYS // B]))

    kc = torch.randn((nblocks, Hkv, B, D), dtype=torch.bfloat16, device=dev)
    vc = torch.randn_like(kc)
    t_tab = torch.from_numpy(tables).to(dev)
    t_ctx = torch.from_numpy(ctx).to(dev)
    scale = 1.0 / math.sqrt(D)
    stream = P.current_stream(dev)
    times = {}
    for name, chunk in (("recomputed", SYS + Q), ("cached", Q)):
        q = torch.randn((S * chunk, Hq, D), dtype=torch.bfloat16, device=dev)
        out = torch.empty((S * chunk, Hq, D), dtype=torch.float32, device=dev)
        qs = torch.arange(0, S * chunk + 1, chunk, dtype=torch.int32, device=dev)

        def call():
            P.pa_prefill(out, q, kc, vc, t_tab, t_ctx, qs, scale, chunk, stream=stream)

        for _ in range(100):    # untimed: lets the matrix-core clock settle (~30-60 ms)
            call()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in evs:
            e0.record()
            call()
            e1.record()
        torch.cuda.synchronize()
        times[name] = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    ctx_l = [SYS + Q] * S
    flops_cached = prefill_flops(ctx_l, list(range(0, S * Q + 1, Q)), D, Hq)
    log(f"[bench] prefix cache: {rounds * S / host_s:.0f} admissions/s; prefill recomputed "
        f"{times['recomputed']:.4f} ms, cached {times['cached']:.4f} ms")
    res = {
        "metric": "prefix cache: batch prefill time with a shared system prompt cached vs recomputed",
        "value": round(times["recomputed"] / times["cached"], 3),
        "unit": "x (recomputed / cached prefill time)",
        "config": {"workload": "16 requests, shared 1024-token system prompt + private 512-token questions",
                   "block_size": B, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D, "kv_dtype": "bf16",
                   "cached_tokens_per_request": cached, "system_blocks_shared": shared // S},
        "prefill_recomputed_ms": round(times["recomputed"], 5),
        "prefill_cached_ms": round(times["cached"], 5),
        "host": {"admissions_per_s": round(rounds * S / host_s, 1),
                 "block_lookups_per_s": round(st["lookups"] / host_s, 1) if host_s > 0 else None,
                 "hit_blocks": st["hit_blocks"], "registered": st["registered"], "evictions": st["evictions"]},
        "roofline": {"bound": "mfma", "kernel": "pa_prefill, cached (512-row chunks)",
                     "achieved": round(flops_cached / (times["cached"] * 1e-3) / 1e12, 2),
                     "peak": PEAK_MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flops_cached / (times["cached"] * 1e-3) / 1e12 / PEAK_MFMA_BF16_TFLOPS, 4),
                     "traffic": None},
        "cpu_baseline": None,
    }
    if with_cpu:
        from oracle.prefix_cache import PrefixPoolModel
        m = PrefixPoolModel(nblocks, B)
        for s in range(S):
            m.alloc_prefix(s, prompts[0][s].tolist(), 7)
        for s in range(S):
            m.free(s)
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 2.0 and n < rounds:
            batch = [prompts[n + 1][s].tolist() for s in range(S)]
            for s in range(S):
                m.alloc_prefix(10 ** 7 + n * S + s, batch[s], 7)
            for s in range(S):
                m.free(10 ** 7 + n * S + s)
            n += 1
        wall = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(n * S / wall, 1), "unit": "admissions/s", "cores": 1,
                               "kind": "oracle", "sample": f"{n} rounds of 16 admissions + releases, {wall:.1f} s"}
    return res


PCIE5_X16_GBPS = 64.0   # one direction, nominal


def bench_swap(dev, with_cpu, seqs=64, tokens=2048, reps=5):
    """Swap copies: preempting `seqs` sequences of `tokens` tokens of the
    Llama-3.1-8B-like GQA layer (8 KV heads, head_dim 128, bf16, B = 16):
    their blocks, scattered over a pool, go to pinned host memory
    (pa_swap_out) and come back into other scattered blocks (pa_swap_in).
    HIP events around each launch; beside them a plain contiguous copy of the
    same bytes between the device and the same pinned buffer (the practical
    ceiling of the host link).  CPU baseline: the layout definition written
    out in numpy (a gather of the same blocks from a host copy of the
    caches)."""
    import numpy as np
    import torch

    import paged_kv_cache_147_amd as P
    Hkv, B, D = 8, 16, 128
    nblk = seqs * tokens // B
    pool_blocks = 2 * nblk + 64
    rng = np.random.default_rng(0)
    perm = rng.permutation(pool_blocks).astype(np.int32)
    out_ids = torch.from_numpy(perm[:nblk].copy()).to(dev)
    in_ids = torch.from_numpy(perm[nblk:2 * nblk].copy()).to(dev)
    kc = torch.randn((pool_blocks, Hkv, B, D), dtype=torch.bfloat16, device=dev)
    vc = torch.randn_like(kc)
    host = torch.empty((nblk, 2, Hkv, B, D), dtype=torch.bfloat16).pin_memory()
    nbytes = host.numel() * host.element_size()
    flat = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev)
    stream = P.current_stream(dev)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in evs:
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs]))

    hflat = host.view(-1)
    t_out = timed(lambda: P.pa_swap_out(kc, vc, out_ids, host, stream=stream))
    t_in = timed(lambda: P.pa_swap_in(kc, vc, in_ids, host, stream=stream))
    t_d2h = timed(lambda: hflat.copy_(flat, non_blocking=True))
    t_h2d = timed(lambda: flat.copy_(hflat, non_blocking=True))
    ok = bool(torch.equal(kc[in_ids.long()].view(torch.int16), kc[out_ids.long()].view(torch.int16)))
    gb = nbytes / 1e9
    log(f"[bench] swap: out {t_out:.3f} ms ({gb / t_out * 1e3:.1f} GB/s), in {t_in:.3f} ms "
        f"({gb / t_in * 1e3:.1f} GB/s); plain copies {gb / t_d2h * 1e3:.1f} / {gb / t_h2d * 1e3:.1f} GB/s")
    res = {
        "metric": "swap-out / swap-in of preempted sequences' blocks: GB/s over the host link",
        "value": round(gb / t_out * 1e3, 2),
        "unit": "GB/s (swap-out)",
        "config": {"workload": f"{seqs} sequences x {tokens} tokens, Llama-3.1-8B-like GQA layer",
                   "num_kv_heads": Hkv, "block_size": B, "head_dim": D, "kv_dtype": "bf16", "blocks": nblk,
                   "bytes": nbytes, "blocks_scattered_over": pool_blocks},
        "swap_out_ms": round(t_out, 4), "swap_in_ms": round(t_in, 4),
        "swap_in_gbps": round(gb / t_in * 1e3, 2),
        "plain_copy_gbps": {"device_to_host": round(gb / t_d2h * 1e3, 2), "host_to_device": round(gb / t_h2d * 1e3, 2)},
        "round_trip_bit_exact": ok,
        "roofline": {"bound": "pcie", "kernel": "pa_swap_out (one launch)", "achieved": round(gb / t_out * 1e3, 2),
                     "peak": PCIE5_X16_GBPS, "unit": "GB/s", "frac": round(gb / t_out * 1e3 / PCIE5_X16_GBPS, 4),
                     "traffic": None},
        "cpu_baseline": None,
    }
    if with_cpu:
        kh, vh = kc.view(torch.int16).cpu().numpy(), vc.view(torch.int16).cpu().numpy()
        ids = out_ids.cpu().numpy()
        dst = np.empty((nblk, 2, Hkv, B, D), dtype=np.int16)
        t0 = time.perf_counter()
        dst[:, 0] = kh[ids]
        dst[:, 1] = vh[ids]
        wall = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(gb / wall, 2), "unit": "GB/s", "cores": 1, "kind": "oracle",
                               "sample": f"numpy gather of the same {nblk} blocks into the documented layout, "
                                         f"host memory to host memory, {wall:.2f} s"}
    return res


FP8_METRIC = "paged decode attention over an E4M3 (FP8) KV cache: KV HBM GB/s (% of MI355X peak)"
FP8_TRAFFIC_WORKLOAD = "llama31_8b_gqa_fp8"


def measured_fp8_traffic(workload):
    """Per-launch HBM bytes of the E4M3 decode from the committed counter
    summary, or None when its source changed since the counters were taken."""
    try:
        text = open(TRAFFIC_FILE, encoding="utf-8").read()
    except OSError:
        return None
    m = re.search(r"^\|\s*" + re.escape(workload) + r"\s*\|\s*([0-9a-f]{16})\s*\|\s*([0-9.e+]+)\s*\|",
                  text, flags=re.M)
    if not m or m.group(1) != source_digest(("decode_fp8.hip", "decode_params.h", "device_common.h")):
        return None
    return float(m.group(2))


def _fp8_chunk(sl):
    from oracle import fp8 as F
    st = _FORK["fp8"]
    F.paged_decode_fp8(st["q"][sl], st["dtype"], st["k"], st["v"], st["ks"], st["vs"], st["tables"][sl],
                       st["lens"][sl], st["B"], st["scale"], st["Hq"], st["Hkv"])


def _shared_u8(shape):
    """A zeroed uint8 array in anonymous shared memory: forked processes
    write into it and the parent sees the result."""
    import mmap

    import numpy as np
    n = int(np.prod(shape))
    return np.frombuffer(mmap.mmap(-1, max(n, 1)), dtype=np.uint8)[:n].reshape(shape)


def _quantize_chunk(sl):
    """E4M3 codes (the oracle's quantisation) of a slice of the used blocks."""
    import numpy as np

    from oracle import fp8 as F
    from oracle.bits import to_f64
    st = _FORK["quant"]
    ids = st["used"][sl]
    st["kc"][ids] = F.quantize(to_f64(st["k"][ids], st["dtype"]).astype(np.float32), st["ks"])
    st["vc"][ids] = F.quantize(to_f64(st["v"][ids], st["dtype"]).astype(np.float32), st["vs"])


def fp8_cpu_baseline(wl, k_scale, v_scale):
    """oracle.fp8.paged_decode_fp8, as it stands, over the whole batch on
    every available core (codes quantised by the oracle beforehand,
    untimed); GB/s of code bytes."""
    import numpy as np

    from oracle import fp8 as F
    from oracle.bits import to_f64
    from tests._replay import OracleRun
    run = OracleRun(wl)
    tables, lens = run.tables(wl)
    used = np.unique(tables[tables >= 0])
    kc, vc = _shared_u8(run.cache.k.shape), _shared_u8(run.cache.v.shape)
    _FORK["quant"] = dict(k=run.cache.k, v=run.cache.v, kc=kc, vc=vc, used=used, dtype=wl.dtype, ks=k_scale,
                          vs=v_scale)
    fork_map(_quantize_chunk, _chunks(len(used), 4 * host_cpu()["cores_available"]), min_wall=0.0, max_reps=1)
    del _FORK["quant"]
    order = np.argsort(-lens, kind="stable")
    _FORK["fp8"] = dict(q=wl.q[order], dtype=wl.dtype, k=kc, v=vc, ks=k_scale, vs=v_scale, tables=tables[order],
                        lens=lens[order], B=wl.block_size, scale=wl.scale, Hq=wl.num_q_heads, Hkv=wl.num_kv_heads)
    cores = host_cpu()["cores_available"]
    wall, cores, reps = fork_map(_fp8_chunk, _chunks(wl.num_seqs, 8 * cores))
    del _FORK["fp8"]
    kv = int(np.sum(lens)) * 2 * wl.num_kv_heads * wl.head_dim
    return {"value": round(kv / wall / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"all {wl.num_seqs} sequences ({kv / 1e9:.3f} GB of codes) on {cores} forked processes, "
                      f"{wall:.2f} s wall (best of {reps}), float64 numpy",
            "seqs_per_s": round(wl.num_seqs / wall, 2), **host_cpu()}


def bench_fp8(wl, run, workload, dev, steps, warmup, nrep, cpu=None, bf16_decode_ms=None,
              k_scale=1 / 56, v_scale=1 / 72, partition_size=0):
    """The decode step over an E4M3 cache: the bf16 cache of the same batch is
    quantised once (pa_write_kv_fp8 over every slot, untimed), then each step
    runs the copy-on-write copies, pa_write_kv_fp8 of the new tokens and
    pa_decode over the codes; pa_decode is timed with HIP events."""
    import numpy as np
    import torch

    import paged_kv_cache_147_amd as P
    nb, hkv, B, d = run.k_cache.shape
    stream = P.current_stream(dev)
    rows_k = run.k_cache.permute(0, 2, 1, 3).reshape(nb * B, hkv, d).contiguous()
    rows_v = run.v_cache.permute(0, 2, 1, 3).reshape(nb * B, hkv, d).contiguous()
    all_slots = torch.arange(nb * B, dtype=torch.int64, device=dev)
    kc = torch.empty((nb, hkv, B, d), dtype=torch.uint8, device=dev)
    vc = torch.empty_like(kc)
    P.pa_write_kv_fp8(kc, vc, rows_k, rows_v, all_slots, k_scale, v_scale, stream=stream)
    del rows_k, rows_v
    replicas = [(kc, vc)] + [(kc.clone(), vc.clone()) for _ in range(nrep - 1)]
    ctx = run.ctx_host.tolist()
    step_rows = torch.cat([torch.arange(r0, r0 + n) for (_, r0, n) in run.step_writes]).to(dev)
    step_slots = torch.cat([sl for (sl, _, _) in run.step_writes])
    k_new = run.k_rows.index_select(0, step_rows).contiguous()
    v_new = run.v_rows.index_select(0, step_rows).contiguous()
    pairs = torch.tensor(run.step_copies, dtype=torch.int32, device=dev) if run.step_copies else None
    out = torch.empty((wl.num_seqs, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device=dev)
    probe = P._lib.decode_args(out, run.q, kc, vc, run.tables, run.ctx, wl.scale, max_ctx=max(ctx),
                               partition_size=partition_size, k_scale=k_scale, v_scale=v_scale)
    ws = P._lib.workspace_for(P.pa_decode_workspace_bytes(probe), dev)

    def step(i, ev=None):
        k, v = replicas[i % len(replicas)]
        if pairs is not None:
            P.pa_copy_blocks(k, v, pairs, stream=stream)
        P.pa_write_kv_fp8(k, v, k_new, v_new, step_slots, k_scale, v_scale, stream=stream)
        if ev is not None:
            ev[0].record()
        P.pa_decode(out, run.q, k, v, run.tables, run.ctx, wl.scale, max_ctx=max(ctx), workspace=ws,
                    partition_size=partition_size, stream=stream, k_scale=k_scale, v_scale=v_scale)
        if ev is not None:
            ev[1].record()

    prewarm = run_prewarm(step)   # untimed, as in bench_decode_step
    for i in range(warmup):
        step(prewarm + i)
    ms_step, dec_ms = timed_passes(step, prewarm + warmup, steps)
    dec_avg = float(np.mean(dec_ms))
    S, Hq = wl.num_seqs, wl.num_q_heads
    kv = int(sum(ctx)) * 2 * hkv * d
    alg = kv + S * Hq * d * 2 + S * Hq * d * 4 + sum(4 * ((c + B - 1) // B) for c in ctx) + 4 * S
    log(f"[bench] fp8: {steps} steps: {ms_step:.4f} ms/step; pa_decode avg {dec_avg:.4f} ms "
        f"(p10 {np.percentile(dec_ms, 10):.4f}, p90 {np.percentile(dec_ms, 90):.4f})")
    gbps = kv / (ms_step * 1e-3) / 1e9
    achieved = alg / (dec_avg * 1e-3) / 1e9
    traffic = measured_fp8_traffic(workload + "_fp8")
    hbm_gbps = traffic / (dec_avg * 1e-3) / 1e9 if traffic else None
    res = {
        "metric": FP8_METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "steps": steps,
        "warmup": warmup,
        "prewarm_steps": prewarm,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "dtype": "fp8_e4m3 codes, bf16 q, f32 accumulation",
        "data": "synthetic",
        "config": {"workload": workload + "_fp8", "batch": S, "num_q_heads": Hq, "num_kv_heads": hkv,
                   "head_dim": d, "block_size": B, "kv_dtype": "fp8_e4m3", "q_dtype": wl.dtype,
                   "out_dtype": "f32", "k_scale": k_scale, "v_scale": v_scale, "partition_size": partition_size,
                   "ctx_mean": round(float(np.mean(ctx)), 1), "kv_bytes_per_step": kv,
                   "cache_replicas": len(replicas)},
        "pct_of_peak": round(100 * gbps / PEAK_HBM_GBPS, 2),
        "seqs_per_s": round(S / (ms_step * 1e-3), 1),
        "decode_speedup_vs_bf16": round(bf16_decode_ms / dec_avg, 3) if bf16_decode_ms else None,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic,
                     "hbm_gbps": round(hbm_gbps, 2) if hbm_gbps else None,
                     "hbm_frac": round(hbm_gbps / PEAK_HBM_GBPS, 4) if hbm_gbps else None,
                     "kernel": "pa_decode over E4M3 codes (partition + combine launches)",
                     "avg_launch_ms": round(dec_avg, 5), "bytes_per_launch": alg,
                     "launch_ms_p10_median_p90": [round(float(np.percentile(dec_ms, q)), 5) for q in (10, 50, 90)]},
        "cpu_baseline": cpu,
    }
    return res


def copy_calibration(dev):
    """Three plain 1 GiB device copies: the reference for the HBM counters."""
    import torch
    a = torch.empty(2 ** 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log("[bench] copy calibration: 3 x 1 GiB device copies done")


def time_calls(fn, n, warm=5):
    """Average duration (ms) of fn() over n calls, HIP events around each."""
    import numpy as np
    import torch
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        evs[i][0].record()
        fn(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in evs]))


def unique_kv_bytes(wl, tables, ctx):
    """KV bytes of the distinct token rows a batch reads (shared prefix
    blocks count once)."""
    import numpy as np
    B = wl.block_size
    slots = []
    for s, c in enumerate(ctx):
        pos = np.arange(int(c))
        slots.append(tables[s, pos // B].astype(np.int64) * B + pos % B)
    n = len(np.unique(np.concatenate(slots))) if slots else 0
    return n * 2 * wl.num_kv_heads * wl.head_dim * elem_bytes(wl.dtype)


def run_prewarm(step):
    """Untimed steps until the GPU's clocks have settled: at least PREWARM_STEPS
    steps and PREWARM_S seconds.  Returns the number of steps run."""
    import torch
    n, t0 = 0, time.perf_counter()
    while n < PREWARM_STEPS or time.perf_counter() - t0 < PREWARM_S:
        for _ in range(10):
            step(n)
            n += 1
        torch.cuda.synchronize()
    return n


def timed_passes(step, first, steps):
    """The timed region: `steps` steps with nothing else on the stream, timed
    by the host clock between two synchronisations (ms per step).  Then the
    same number of steps again with HIP events recorded around the measured
    call of each (step(i, events)), which give the roofline's launch
    durations.  The event records are kept out of the first pass: on this
    stack two records per step add ~6.5 us to the step time while the
    durations they measure are unchanged.  Returns (ms per step, per-call ms
    from the events)."""
    import torch
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(steps):
        step(first + i)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t_start) * 1e3 / steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        step(first + steps + i, evs[i])
    torch.cuda.synchronize()
    return ms_step, [a.elapsed_time(b) for a, b in evs]


def bench_decode_step(wl, workload, desc, dev, steps, warmup, nrep, partition_size=0, cpu=None):
    """One decode step (copies, pa_write_kv of the new tokens, pa_decode),
    timed over `steps` steps after `warmup`, then `steps` more with every
    pa_decode call between HIP events on the stream it runs on
    (timed_passes).  Returns (result, device run, average pa_decode ms)."""
    import numpy as np
    import torch

    import paged_kv_cache_147_amd as P
    from tests._native import NativeDeviceRun
    t0 = time.time()
    run = NativeDeviceRun(wl, device=dev)
    ctx = run.ctx_host.tolist()
    kv_bytes, alg_bytes = decode_bytes(wl, ctx)
    uniq = unique_kv_bytes(wl, run.tables.cpu().numpy(), ctx)
    log(f"[bench] {workload}: cache built in {time.time() - t0:.1f}s; {wl.num_seqs} seqs, KV {kv_bytes / 1e9:.3f} GB "
        f"logical, {uniq / 1e9:.3f} GB unique")
    step_rows = torch.cat([torch.arange(r0, r0 + n) for (_, r0, n) in run.step_writes]).to(dev)
    step_slots = torch.cat([s for (s, _, _) in run.step_writes])
    k_new = run.k_rows.index_select(0, step_rows).contiguous()
    v_new = run.v_rows.index_select(0, step_rows).contiguous()
    pairs = (torch.tensor(run.step_copies, dtype=torch.int32, device=dev) if run.step_copies else None)
    replicas = [(run.k_cache, run.v_cache)]
    for _ in range(nrep - 1):
        replicas.append((run.k_cache.clone(), run.v_cache.clone()))
    out = torch.empty((wl.num_seqs, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device=dev)
    probe = P._lib.decode_args(out, run.q, run.k_cache, run.v_cache, run.tables, run.ctx, wl.scale,
                               max_ctx=max(ctx), partition_size=partition_size)
    ws = P._lib.workspace_for(P.pa_decode_workspace_bytes(probe), dev)
    stream = P.current_stream(dev)

    def step(i, ev=None):
        kc, vc = replicas[i % len(replicas)]
        if pairs is not None:
            P.pa_copy_blocks(kc, vc, pairs, stream=stream)
        P.pa_write_kv(kc, vc, k_new, v_new, step_slots, stream=stream)
        if ev is not None:
            ev[0].record()
        P.pa_decode(out, run.q, kc, vc, run.tables, run.ctx, wl.scale, max_ctx=max(ctx),
                    partition_size=partition_size, workspace=ws, stream=stream)
        if ev is not None:
            ev[1].record()

    # Untimed pre-warm before the W warmup steps: the GPU's clocks take tens of
    # milliseconds of load to settle, and a short timed run (the default
    # --steps 20 --warmup 5 is ~5 ms of decode) would otherwise read part of
    # that ramp.
    prewarm = run_prewarm(step)
    for i in range(warmup):
        step(prewarm + i)
    ms_step, dec_ms = timed_passes(step, prewarm + warmup, steps)
    dec_avg = float(np.mean(dec_ms))
    log(f"[bench] {workload}: {steps} steps: {ms_step:.4f} ms/step; pa_decode avg {dec_avg:.4f} ms "
        f"(p10 {np.percentile(dec_ms, 10):.4f}, p90 {np.percentile(dec_ms, 90):.4f})")
    gbps = kv_bytes / (ms_step * 1e-3) / 1e9
    achieved = alg_bytes / (dec_avg * 1e-3) / 1e9
    traffic = measured_traffic(workload)
    hbm_gbps = traffic / (dec_avg * 1e-3) / 1e9 if traffic else None
    res = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "steps": steps,
        "warmup": warmup,
        "prewarm_steps": prewarm,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "accumulate": "f32",
        "data": "synthetic",
        "config": {"workload": workload, "description": desc, "batch": wl.num_seqs,
                   "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads,
                   "head_dim": wl.head_dim, "block_size": wl.block_size, "kv_dtype": wl.dtype,
                   "out_dtype": "f32", "ctx_mean": round(float(np.mean(ctx)), 1),
                   "ctx_max": int(max(ctx)), "kv_bytes_per_step": kv_bytes, "unique_kv_bytes_per_step": uniq,
                   "cache_replicas": len(replicas), "partition_size": partition_size,
                   "parallelism": "single GPU"},
        "logical_kv_gbps": round(gbps, 2),
        "pct_of_peak": round(100 * gbps / PEAK_HBM_GBPS, 2),
        "seqs_per_s": round(wl.num_seqs / (ms_step * 1e-3), 1),
        "decode_seqs_per_s": round(wl.num_seqs / (dec_avg * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic,
                     "hbm_gbps": round(hbm_gbps, 2) if hbm_gbps else None,
                     "hbm_frac": round(hbm_gbps / PEAK_HBM_GBPS, 4) if hbm_gbps else None,
                     "unique_kv_gbps": round(uniq / (dec_avg * 1e-3) / 1e9, 2),
                     "kernel": "pa_decode (partition + combine launches)",
                     "avg_launch_ms": round(dec_avg, 5), "bytes_per_launch": alg_bytes,
                     "launch_ms_p10_median_p90": [round(float(np.percentile(dec_ms, q)), 5) for q in (10, 50, 90)]},
        "cpu_baseline": cpu,
    }
    del replicas
    return res, run, dec_avg


def time_contiguous(wl, run, steps, nrep, dev, partition_size=0):
    """pa_decode vs the same attention on the contiguous layout (identical
    logical K/V), and vs the paged kernel with its blocks placed in table
    order (identity free list: the same lookups over contiguous memory); all
    three timed alike (the decode call alone, rotating cache copies)."""
    import numpy as np
    import torch

    import paged_kv_cache_147_amd as P
    from tests._native import NativeDeviceRun, device_tensor
    from tests._replay import contiguous_layout
    stream = P.current_stream(dev)
    ctx = run.ctx_host
    mctx = int(ctx.max())
    out = torch.empty((wl.num_seqs, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device=dev)
    reps = [(run.k_cache, run.v_cache)] + [(run.k_cache.clone(), run.v_cache.clone()) for _ in range(nrep - 1)]
    ws = [None]

    def paged(i):
        kc, vc = reps[i % len(reps)]
        ws[0] = P.pa_decode(out, run.q, kc, vc, run.tables, run.ctx, wl.scale, max_ctx=mctx,
                            partition_size=partition_size, workspace=ws[0], stream=stream)
    paged_ms = time_calls(paged, steps)
    del reps
    cap = (mctx + 7) // 8 * 8
    k, v, _ = contiguous_layout(wl, capacity=cap)
    creps = [(device_tensor(k, wl.dtype, dev), device_tensor(v, wl.dtype, dev))]
    del k, v
    creps += [(creps[0][0].clone(), creps[0][1].clone()) for _ in range(nrep - 1)]
    wsc = [None]

    def contig(i):
        kc, vc = creps[i % len(creps)]
        wsc[0] = P.pa_decode_contiguous(out, run.q, kc, vc, run.ctx, wl.scale, max_ctx=mctx,
                                        partition_size=partition_size, workspace=wsc[0], stream=stream)
    contig_ms = time_calls(contig, steps)
    del creps
    wl_id = type(wl)(**{**wl.__dict__, "free_order": np.arange(wl.num_blocks, dtype=np.int32)})
    run_id = NativeDeviceRun(wl_id, device=dev)
    ireps = [(run_id.k_cache, run_id.v_cache)] + [(run_id.k_cache.clone(), run_id.v_cache.clone())
                                                 for _ in range(nrep - 1)]
    wsi = [None]

    def paged_identity(i):
        kc, vc = ireps[i % len(ireps)]
        wsi[0] = P.pa_decode(out, run_id.q, kc, vc, run_id.tables, run_id.ctx, wl.scale, max_ctx=mctx,
                             partition_size=partition_size, workspace=wsi[0], stream=stream)
    ident_ms = time_calls(paged_identity, steps)
    del ireps, run_id
    return {"paged_ms": round(paged_ms, 5), "contiguous_ms": round(contig_ms, 5),
            "paged_identity_placement_ms": round(ident_ms, 5),
            "overhead_vs_contiguous": round(paged_ms / contig_ms - 1, 4),
            "overhead_identity_vs_contiguous": round(ident_ms / contig_ms - 1, 4)}


def bench_configs(dev, steps, warmup, nrep):
    """The other decode configurations of the scope, each a full step (copies,
    pa_write_kv, pa_decode) at its real size: the Llama-7B-like MHA layer, the
    LLaMA-13B-like layer at context 4096, and its 4-beam batch with the step's
    copy-on-write copies.  Same timing as the headline line."""
    import torch

    import workloads as W
    out = {}
    for name in ("llama7b_mha", "llama13b_long", "llama13b_beam"):
        key, desc = WORKLOADS[name]
        wl = W.CONFIGS[key]()
        res, run, _ = bench_decode_step(wl, name, desc, dev, steps, warmup, nrep)
        del run
        torch.cuda.empty_cache()
        r = res["roofline"]
        out[name] = {"description": desc, "batch": wl.num_seqs, "heads": [wl.num_q_heads, wl.num_kv_heads],
                     "kv_dtype": wl.dtype, "ctx_mean": res["config"]["ctx_mean"],
                     "kv_bytes_per_step": res["config"]["kv_bytes_per_step"],
                     "ms_per_step": res["ms_per_step"], "step_gbps": res["value"], "seqs_per_s": res["seqs_per_s"],
                     "decode_ms": r["avg_launch_ms"], "decode_seqs_per_s": res["decode_seqs_per_s"],
                     "roofline": {k: r[k] for k in ("bound", "achieved", "peak", "unit", "frac")}}
    return out


def bench_block_sweep(dev, steps, nrep):
    """Block sizes 8 / 16 / 32 on 128 sequences at ctx 1000 (GQA 32 / 8, d 128,
    bf16, identical logical Q/K/V for every B): the paged call, the
    contiguous-layout call and the identity-placement call, decode only."""
    import torch

    import workloads as W
    rows = {}
    for B in (8, 16, 32):
        wl = W.block_sweep(B)
        from tests._native import NativeDeviceRun
        run = NativeDeviceRun(wl, device=dev)
        kv, alg = decode_bytes(wl, run.ctx_host.tolist())
        r = time_contiguous(wl, run, steps, nrep, dev)
        r["paged_gbps"] = round(alg / (r["paged_ms"] * 1e-3) / 1e9, 2)
        r["paged_frac"] = round(alg / (r["paged_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)
        r["contiguous_gbps"] = round(alg / (r["contiguous_ms"] * 1e-3) / 1e9, 2)
        r["blocks_per_seq"] = -(-1000 // B)
        rows[f"B{B}"] = r
        log(f"[bench] block sweep B={B}: paged {r['paged_ms']:.4f} ms, contiguous {r['contiguous_ms']:.4f} ms, "
            f"identity {r['paged_identity_placement_ms']:.4f} ms ({100 * r['overhead_vs_contiguous']:+.1f}%)")
        del run
        torch.cuda.empty_cache()
    return {"metric": "paged vs contiguous-layout pa_decode time (indirection overhead)",
            "config": {"workload": "ctx 1000 x 128 sequences, GQA 32/8, d 128, bf16, B in {8, 16, 32}",
                       "kv_bytes_per_call": kv, "calls_timed": steps, "cache_replicas": nrep},
            **rows}


def bench_ceiling(dev, reps=20):
    """Read rates this GPU reaches with no arithmetic: a plain stream over
    1 GiB, and whole 4 KiB tiles at scattered indices of a 4 GiB buffer
    (the decode's (block, KV head) tile shape), 1 GiB read per launch; HIP
    events around each launch.  Each with the default and with the
    non-temporal cache policy (the one the decode uses for unshared rows)."""
    import ctypes

    import numpy as np
    import torch

    import paged_kv_cache_147_amd as P
    lib = ctypes.CDLL(os.path.join(ROOT, "paged_kv_cache_147_amd", "libpagedkv_ceiling.so"))
    lib.pc_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int,
                                   ctypes.c_void_p]
    lib.pc_tile_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int,
                                 ctypes.c_void_p]
    stream = P.current_stream(dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    nbytes = 1 << 30
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device=dev), torch.full((nbytes,), 3, dtype=torch.uint8, device=dev)]
    blocks = cus * 8
    sink = torch.empty(blocks * 256 * 16, dtype=torch.uint8, device=dev)

    def timed(fn):
        fn(0)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for i, (e0, e1) in enumerate(evs):
            e0.record()
            fn(i)
            e1.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in evs]))

    def stream_read(i, nt=0):
        assert lib.pc_stream_read(bufs[i % 2].data_ptr(), nbytes, blocks, sink.data_ptr(), nt, stream) == 0
    ms_stream = timed(stream_read)
    ms_stream_nt = timed(lambda i: stream_read(i, 1))
    del bufs
    tile = 4096
    big = torch.ones(4 * nbytes, dtype=torch.uint8, device=dev)
    n_tiles = nbytes // tile
    rng = np.random.default_rng(0)
    ids = [torch.from_numpy(rng.permutation(4 * nbytes // tile)[:n_tiles].astype(np.int32)).to(dev) for _ in range(2)]
    per_wave = 16
    tsink = torch.empty(-(-n_tiles // per_wave) * 64 * 16, dtype=torch.uint8, device=dev)

    def tile_read(i, nt=0):
        assert lib.pc_tile_read(big.data_ptr(), ids[i % 2].data_ptr(), n_tiles, tsink.data_ptr(), nt, stream) == 0
    ms_tile = timed(tile_read)
    ms_tile_nt = timed(lambda i: tile_read(i, 1))
    del big
    torch.cuda.empty_cache()
    res = {"metric": "read rate with no arithmetic (context for the decode roofline)",
           "unit": "GB/s", "peak": PEAK_HBM_GBPS,
           "stream_read_gbps": round(nbytes / (ms_stream * 1e-3) / 1e9, 1),
           "stream_read_frac": round(nbytes / (ms_stream * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
           "tile4k_read_gbps": round(nbytes / (ms_tile * 1e-3) / 1e9, 1),
           "tile4k_read_frac": round(nbytes / (ms_tile * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
           "stream_read_nt_gbps": round(nbytes / (ms_stream_nt * 1e-3) / 1e9, 1),
           "stream_read_nt_frac": round(nbytes / (ms_stream_nt * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
           "tile4k_read_nt_gbps": round(nbytes / (ms_tile_nt * 1e-3) / 1e9, 1),
           "tile4k_read_nt_frac": round(nbytes / (ms_tile_nt * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
           "config": {"stream": f"1 GiB, {blocks} workgroups of 256 threads, one 16-byte load per thread and "
                                "iteration, 2 buffers alternated",
                      "tile4k": f"{n_tiles} 4 KiB tiles at random distinct indices of a 4 GiB buffer, {per_wave} "
                                "tiles per 64-lane wave (4 in flight), 2 index sets alternated",
                      "nt": "the _nt figures load with the non-temporal cache policy",
                      "timing": f"median of {reps} launches, HIP events"}}
    log(f"[bench] ceiling: stream {res['stream_read_gbps']} / {res['stream_read_nt_gbps']} (nt) GB/s, "
        f"4 KiB tiles {res['tile4k_read_gbps']} / {res['tile4k_read_nt_gbps']} (nt) GB/s")
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama31_8b_gqa", choices=sorted(WORKLOADS))
    ap.add_argument("--replicas", type=int, default=4, help="cache copies rotated over steps")
    ap.add_argument("--partition-size", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", choices=("decode", "prefill", "prefix", "swap", "fp8", "ceiling"), default="decode",
                    help="print only one measurement")
    ap.add_argument("--no-extras", "--no-prefill", dest="no_extras", action="store_true",
                    help="decode line only: leave out the nested objects")
    ap.add_argument("--prefill-steps", type=int, default=50)
    ap.add_argument("--prefill-warmup", type=int, default=200,
                    help="untimed pa_prefill launches before the timed ones (~60 ms: the matrix-core "
                         "clock takes that long to settle; 10 launches read ~15%% slow)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--compare-contiguous", action="store_true",
                    help="also time pa_decode_contiguous and identity placement on the chosen workload")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only; multi-GPU runs are not part of it "
              "(use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch  # noqa: F401  (CPU work first: nothing below initialises the GPU until the oracle legs are done)

    import workloads as W
    mode, extras, with_cpu = args.mode, not args.no_extras, not args.no_cpu_baseline
    key, desc = WORKLOADS[args.workload]
    wl = wl_ns = wl_pf = None
    t0 = time.time()
    if mode in ("decode", "fp8"):
        wl = W.CONFIGS[key]()
        if mode == "decode" and extras and args.workload == "llama31_8b_gqa":
            wl_ns = W.CONFIGS["gqa_noshare"]()
    if mode == "prefill" or (mode == "decode" and extras):
        wl_pf = W.llama31_8b_prefill()
    log(f"[bench] workloads generated in {time.time() - t0:.1f}s")
    cpu = {}
    if with_cpu:
        t0 = time.time()
        if mode == "decode":
            cpu["decode"] = cpu_baseline(wl)
            if wl_ns is not None:
                cpu["noshare"] = cpu_baseline(wl_ns)
        if mode == "fp8" or (mode == "decode" and extras):
            cpu["fp8"] = fp8_cpu_baseline(wl, 1 / 56, 1 / 72)
        if wl_pf is not None:
            cpu["prefill"] = prefill_cpu_baseline(wl_pf)
        log(f"[bench] oracle baselines on {host_cpu()['cores_available']} cores in {time.time() - t0:.1f}s")

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    tail = {"n_gpus": 1, "vs_baseline": None}
    if mode == "swap":
        print(json.dumps({**bench_swap(dev, with_cpu), **tail}), flush=True)
        return
    if mode == "prefix":
        print(json.dumps({**bench_prefix(dev, with_cpu), **tail}), flush=True)
        return
    if mode == "ceiling":
        print(json.dumps({**bench_ceiling(dev), **tail}), flush=True)
        return
    if mode == "prefill":
        res = bench_prefill(wl_pf, args.prefill_steps, args.prefill_warmup, dev, cpu.get("prefill"))
        if args.copy_calibration:
            copy_calibration(dev)
        print(json.dumps({**res, "scaling": "weak", **tail}), flush=True)
        return
    if mode == "fp8":
        from tests._native import NativeDeviceRun
        run = NativeDeviceRun(wl, device=dev)
        res = bench_fp8(wl, run, args.workload, dev, args.steps, args.warmup, args.replicas, cpu.get("fp8"),
                        partition_size=args.partition_size)
        if args.copy_calibration:
            copy_calibration(dev)
        print(json.dumps({**res, "scaling": "weak", **tail}), flush=True)
        return

    result, run, dec_avg = bench_decode_step(wl, args.workload, desc, dev, args.steps, args.warmup, args.replicas,
                                             args.partition_size, cpu.get("decode"))
    result["n_gpus"] = 1
    if args.copy_calibration:
        copy_calibration(dev)
    if args.compare_contiguous:
        result["paged_vs_contiguous"] = time_contiguous(wl, run, args.steps, args.replicas, dev,
                                                        args.partition_size)
    if extras:
        if wl_ns is not None:
            ns, run_ns, _ = bench_decode_step(wl_ns, "llama31_8b_gqa_noshare", WORKLOADS["llama31_8b_gqa_noshare"][1],
                                              dev, args.steps, args.warmup, args.replicas, args.partition_size,
                                              cpu.get("noshare"))
            del run_ns
            for k in ("metric", "steps", "warmup", "higher_is_better", "scaling", "vs_baseline", "data"):
                ns.pop(k, None)
            result["noshare"] = ns
            torch.cuda.empty_cache()
        result["fp8"] = bench_fp8(wl, run, args.workload, dev, args.steps, args.warmup, args.replicas,
                                  cpu.get("fp8"), bf16_decode_ms=dec_avg)
        del run
        torch.cuda.empty_cache()
        result["configs"] = bench_configs(dev, min(max(args.steps, 20), 100), args.warmup, args.replicas)
        result["block_sweep"] = bench_block_sweep(dev, max(args.steps, 50), args.replicas)
        result["ceiling"] = bench_ceiling(dev)
        result["prefill"] = bench_prefill(wl_pf, args.prefill_steps, args.prefill_warmup, dev, cpu.get("prefill"))
        result["prefix_cache"] = bench_prefix(dev, with_cpu)
        result["swap"] = bench_swap(dev, with_cpu)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
