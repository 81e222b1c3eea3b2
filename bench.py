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
/ step time (GB/s).  ``roofline`` is measured live with HIP events around
every pa_decode launch in the timed region; ``cpu_baseline`` times the float64
oracle on a bounded sample of the same batch.

The line also carries a ``prefill`` object: pa_prefill (chunked causal
prefill over the paged cache) on the Llama-3.1-8B-like prefill batch (16
sequences, 512-token chunks after cached prefixes of 0..2048 tokens), in
algorithmic TFLOP/s against the dense bf16 matrix-core peak, with its own
roofline and oracle baseline.  ``--mode prefill`` prints that object alone.
``prefix_cache`` and ``swap`` measure the prefix cache and the preemption
copies; ``fp8`` runs the same decode step over an E4M3 copy of the cache
(pa_write_kv_fp8 of the new tokens, pa_decode over codes), with its own
roofline and oracle baseline.  ``--mode prefix|swap|fp8`` prints one alone.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--mode decode|prefill|prefix|swap|fp8] [--no-prefill]
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
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "paged_kv_cache_147_amd", "csrc", name), "rb") as f:
            h.update(f.read())
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


def cpu_baseline(wl, budget_s=10.0):
    """The float64 oracle, as it stands, on the first sequences of the batch
    until ~budget_s of work; scaled to GB/s of logical KV."""
    import numpy as np

    from oracle import attention as A
    from tests._replay import OracleRun
    run = OracleRun(wl)
    tables, lens = run.tables(wl)
    e = elem_bytes(wl.dtype)
    done, kv, wall, cpu = 0, 0, 0.0, 0.0
    while done < wl.num_seqs and wall < budget_s:
        n = min(8, wl.num_seqs - done)
        sl = slice(done, done + n)
        t0, c0 = time.perf_counter(), time.process_time()
        A.paged_decode(wl.q[sl], run.cache.k, run.cache.v, tables[sl], lens[sl], wl.block_size,
                       wl.scale, wl.dtype, wl.num_q_heads, wl.num_kv_heads)
        wall += time.perf_counter() - t0
        cpu += time.process_time() - c0
        kv += int(np.sum(lens[sl])) * 2 * wl.num_kv_heads * wl.head_dim * e
        done += n
    return {"value": round(kv / wall / 1e9, 4), "unit": "GB/s", "cores": max(1, round(cpu / wall)),
            "kind": "oracle",
            "sample": f"first {done} of {wl.num_seqs} sequences ({kv / 1e9:.3f} GB logical KV), "
                      f"{wall:.1f} s wall, float64 numpy",
            "seqs_per_s": round(done / wall, 2), **host_cpu()}


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


def prefill_cpu_baseline(wl, budget_s=10.0):
    """The float64 prefill oracle, as it stands, on whole sequences of the
    batch (all rows, all heads) until ~budget_s of work; in TFLOP/s."""
    import numpy as np

    from oracle import prefill as PF
    from tests._replay import OracleRun
    run = OracleRun(wl)
    tables, lens = run.tables(wl)
    qs = wl.info["q_start"]
    done, flops, wall, cpu = 0, 0, 0.0, 0.0
    while done < wl.num_seqs and wall < budget_s:
        s = done
        rows = [(r, h) for r in range(qs[s], qs[s + 1]) for h in range(wl.num_q_heads)]
        t0, c0 = time.perf_counter(), time.process_time()
        PF.paged_prefill(wl.info["q_rows"], run.cache.k, run.cache.v, tables, lens, qs, wl.block_size,
                         wl.scale, wl.dtype, wl.num_q_heads, wl.num_kv_heads, rows=rows)
        wall += time.perf_counter() - t0
        cpu += time.process_time() - c0
        flops += prefill_flops(lens[s:s + 1], [0, qs[s + 1] - qs[s]], wl.head_dim, wl.num_q_heads)
        done += 1
    return {"value": round(flops / wall / 1e12, 6), "unit": "TFLOP/s", "cores": max(1, round(cpu / wall)),
            "kind": "oracle",
            "sample": f"first {done} of {wl.num_seqs} sequences, every chunk row and head "
                      f"({flops / 1e9:.2f} GFLOP), {wall:.1f} s wall, float64 numpy", **host_cpu()}


def bench_prefill(steps, warmup, dev, with_cpu):
    """pa_prefill on the Llama-3.1-8B-like prefill batch: each launch timed
    with HIP events on the stream it runs on."""
    import numpy as np
    import torch

    import paged_kv_cache_147_amd as P
    import workloads as W
    from tests._native import NativeDeviceRun, device_tensor
    wl = W.llama31_8b_prefill()
    run = NativeDeviceRun(wl, device=dev)
    ctx = run.ctx_host.tolist()
    qs = [int(x) for x in wl.info["q_start"]]
    q = device_tensor(wl.info["q_rows"], wl.dtype, dev)
    q_start = torch.tensor(qs, dtype=torch.int32, device=dev)
    max_chunk = int(max(wl.info["chunk"]))
    out = torch.empty((q.shape[0], wl.num_q_heads, wl.head_dim), dtype=torch.float32, device=dev)
    stream = P.current_stream(dev)
    flops = prefill_flops(ctx, qs, wl.head_dim, wl.num_q_heads)

    def call():
        P.pa_prefill(out, q, run.k_cache, run.v_cache, run.tables, run.ctx, q_start, wl.scale, max_chunk,
                     stream=stream)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t_start = time.perf_counter()
    for e0, e1 in evs:
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms = [a.elapsed_time(b) for a, b in evs]
    ms_call = elapsed * 1e3 / steps
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
        "cpu_baseline": None,
    }
    if with_cpu:
        log("[bench] timing the prefill oracle on a CPU sample ...")
        res["cpu_baseline"] = prefill_cpu_baseline(wl)
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


def fp8_cpu_baseline(wl, k_scale, v_scale, budget_s=10.0):
    """oracle.fp8.paged_decode_fp8, as it stands, on the first sequences of the
    batch until ~budget_s of work (codes quantised by the oracle beforehand,
    untimed); scaled to GB/s of code bytes."""
    import numpy as np

    from oracle import fp8 as F
    from oracle.bits import to_f64
    from tests._replay import OracleRun
    run = OracleRun(wl)
    tables, lens = run.tables(wl)
    kc = F.quantize(to_f64(run.cache.k, wl.dtype).astype(np.float32), k_scale)
    vc = F.quantize(to_f64(run.cache.v, wl.dtype).astype(np.float32), v_scale)
    done, kv, wall, cpu = 0, 0, 0.0, 0.0
    while done < wl.num_seqs and wall < budget_s:
        n = min(8, wl.num_seqs - done)
        sl = slice(done, done + n)
        t0, c0 = time.perf_counter(), time.process_time()
        F.paged_decode_fp8(wl.q[sl], wl.dtype, kc, vc, k_scale, v_scale, tables[sl], lens[sl], wl.block_size,
                           wl.scale, wl.num_q_heads, wl.num_kv_heads)
        wall += time.perf_counter() - t0
        cpu += time.process_time() - c0
        kv += int(np.sum(lens[sl])) * 2 * wl.num_kv_heads * wl.head_dim
        done += n
    return {"value": round(kv / wall / 1e9, 4), "unit": "GB/s", "cores": max(1, round(cpu / wall)),
            "kind": "oracle",
            "sample": f"first {done} of {wl.num_seqs} sequences ({kv / 1e9:.3f} GB of codes), "
                      f"{wall:.1f} s wall, float64 numpy",
            "seqs_per_s": round(done / wall, 2), **host_cpu()}


def bench_fp8(wl, run, workload, dev, steps, warmup, nrep, with_cpu, bf16_decode_ms=None,
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

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t_start = time.perf_counter()
    for i in range(steps):
        step(warmup + i, evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    dec_ms = [a.elapsed_time(b) for a, b in evs]
    ms_step = elapsed * 1e3 / steps
    dec_avg = float(np.mean(dec_ms))
    S, Hq = wl.num_seqs, wl.num_q_heads
    kv = int(sum(ctx)) * 2 * hkv * d
    alg = kv + S * Hq * d * 2 + S * Hq * d * 4 + sum(4 * ((c + B - 1) // B) for c in ctx) + 4 * S
    log(f"[bench] fp8: {steps} steps: {ms_step:.4f} ms/step; pa_decode avg {dec_avg:.4f} ms "
        f"(p10 {np.percentile(dec_ms, 10):.4f}, p90 {np.percentile(dec_ms, 90):.4f})")
    gbps = kv / (ms_step * 1e-3) / 1e9
    achieved = alg / (dec_avg * 1e-3) / 1e9
    res = {
        "metric": FP8_METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "steps": steps,
        "warmup": warmup,
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
                     "traffic": measured_fp8_traffic(workload + "_fp8"),
                     "kernel": "pa_decode over E4M3 codes (partition + combine launches)",
                     "avg_launch_ms": round(dec_avg, 5), "bytes_per_launch": alg,
                     "launch_ms_p10_median_p90": [round(float(np.percentile(dec_ms, q)), 5) for q in (10, 50, 90)]},
        "cpu_baseline": None,
    }
    if with_cpu:
        log("[bench] timing the E4M3 oracle on a CPU sample ...")
        res["cpu_baseline"] = fp8_cpu_baseline(wl, k_scale, v_scale)
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


def compare_contiguous(wl, run, replicas, ws_paged, args, stream):
    """Paged decode vs the same attention on the contiguous layout (identical
    logical K/V), and vs the paged kernel with blocks placed in order; all
    three timed the same way (pa_decode* alone, rotating cache copies)."""
    import numpy as np
    import torch

    import paged_kv_cache_147_amd as P
    from tests._native import NativeDeviceRun, device_tensor
    from tests._replay import contiguous_layout
    dev = run.q.device
    ctx = run.ctx_host
    cap = int((ctx.max() + 7) // 8 * 8)
    k, v, _ = contiguous_layout(wl, capacity=cap)
    reps = [(device_tensor(k, wl.dtype, dev), device_tensor(v, wl.dtype, dev))]
    for _ in range(args.replicas - 1):
        reps.append((reps[0][0].clone(), reps[0][1].clone()))
    out = torch.empty((wl.num_seqs, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device=dev)
    ws = [None]

    def paged(i):
        kc, vc = replicas[i % len(replicas)]
        P.pa_decode(out, run.q, kc, vc, run.tables, run.ctx, wl.scale, max_ctx=int(ctx.max()),
                    partition_size=args.partition_size, workspace=ws_paged, stream=stream)
    paged_ms = time_calls(paged, args.steps)

    def contig(i):
        kc, vc = reps[i % len(reps)]
        ws[0] = P.pa_decode_contiguous(out, run.q, kc, vc, run.ctx, wl.scale, max_ctx=int(ctx.max()),
                                       partition_size=args.partition_size, workspace=ws[0], stream=stream)
    contig_ms = time_calls(contig, args.steps)
    del reps
    # paged kernel, blocks in table order (free list 0..n-1): same lookups, contiguous placement
    wl_id = type(wl)(**{**wl.__dict__, "free_order": np.arange(wl.num_blocks, dtype=np.int32)})
    run_id = NativeDeviceRun(wl_id, device=dev)
    reps_id = [(run_id.k_cache, run_id.v_cache)] + [(run_id.k_cache.clone(), run_id.v_cache.clone())
                                                   for _ in range(args.replicas - 1)]
    ws_id = [None]

    def paged_identity(i):
        kc, vc = reps_id[i % len(reps_id)]
        ws_id[0] = P.pa_decode(out, run_id.q, kc, vc, run_id.tables, run_id.ctx, wl.scale,
                               max_ctx=int(ctx.max()), partition_size=args.partition_size,
                               workspace=ws_id[0], stream=stream)
    ident_ms = time_calls(paged_identity, args.steps)
    return {"paged_ms": round(paged_ms, 5), "contiguous_ms": round(contig_ms, 5),
            "paged_identity_placement_ms": round(ident_ms, 5),
            "overhead_vs_contiguous": round(paged_ms / contig_ms - 1, 4),
            "overhead_identity_vs_contiguous": round(ident_ms / contig_ms - 1, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama31_8b_gqa", choices=sorted(WORKLOADS))
    ap.add_argument("--replicas", type=int, default=4, help="cache copies rotated over steps")
    ap.add_argument("--partition-size", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", choices=("decode", "prefill", "prefix", "swap", "fp8"), default="decode",
                    help="prefill / prefix: print only the pa_prefill / prefix-cache measurement")
    ap.add_argument("--no-prefill", action="store_true",
                    help="leave the prefill, prefix-cache, swap and fp8 objects out")
    ap.add_argument("--prefill-steps", type=int, default=50)
    ap.add_argument("--prefill-warmup", type=int, default=200,
                    help="untimed pa_prefill launches before the timed ones (~60 ms: the matrix-core "
                         "clock takes that long to settle; 10 launches read ~15%% slow)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--compare-contiguous", action="store_true",
                    help="also time pa_decode_contiguous on the same logical K/V and the paged "
                         "kernel with blocks placed in order (identity free list); adds a "
                         "'paged_vs_contiguous' object to the JSON line")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only; multi-GPU runs are not part of it "
              "(use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_147_amd as P
    import workloads as W
    from tests._native import NativeDeviceRun

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.mode == "swap":
        res = bench_swap(dev, not args.no_cpu_baseline)
        res.update({"n_gpus": 1, "vs_baseline": None})
        print(json.dumps(res), flush=True)
        return
    if args.mode == "prefix":
        res = bench_prefix(dev, not args.no_cpu_baseline)
        res.update({"n_gpus": 1, "vs_baseline": None})
        print(json.dumps(res), flush=True)
        return
    if args.mode == "prefill":
        res = bench_prefill(args.prefill_steps, args.prefill_warmup, dev, not args.no_cpu_baseline)
        if args.copy_calibration:
            copy_calibration(dev)
        res.update({"n_gpus": 1, "scaling": "weak", "vs_baseline": None})
        print(json.dumps(res), flush=True)
        return
    key, desc = WORKLOADS[args.workload]
    t0 = time.time()
    wl = W.CONFIGS[key]()
    log(f"[bench] workload {wl.name}: generated in {time.time() - t0:.1f}s")
    run = NativeDeviceRun(wl, device=dev)
    ctx = run.ctx_host.tolist()
    kv_bytes, alg_bytes = decode_bytes(wl, ctx)
    log(f"[bench] cache built; {wl.num_seqs} seqs, KV {kv_bytes / 1e9:.3f} GB logical")
    if args.mode == "fp8":
        res = bench_fp8(wl, run, args.workload, dev, args.steps, args.warmup, args.replicas,
                        not args.no_cpu_baseline, partition_size=args.partition_size)
        if args.copy_calibration:
            copy_calibration(dev)
        res.update({"n_gpus": 1, "scaling": "weak", "vs_baseline": None})
        print(json.dumps(res), flush=True)
        return

    # The step's own work: copies, then one write of every new token.
    step_rows = torch.cat([torch.arange(r0, r0 + n) for (_, r0, n) in run.step_writes]).to(dev)
    step_slots = torch.cat([s for (s, _, _) in run.step_writes])
    k_new = run.k_rows.index_select(0, step_rows).contiguous()
    v_new = run.v_rows.index_select(0, step_rows).contiguous()
    pairs = (torch.tensor(run.step_copies, dtype=torch.int32, device=dev)
             if run.step_copies else None)
    replicas = [(run.k_cache, run.v_cache)]
    for _ in range(args.replicas - 1):
        replicas.append((run.k_cache.clone(), run.v_cache.clone()))
    out = torch.empty((wl.num_seqs, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device=dev)
    probe = P._lib.decode_args(out, run.q, run.k_cache, run.v_cache, run.tables, run.ctx, wl.scale,
                               max_ctx=max(ctx), partition_size=args.partition_size)
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
                    partition_size=args.partition_size, workspace=ws, stream=stream)
        if ev is not None:
            ev[1].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    dec_ms = [a.elapsed_time(b) for a, b in evs]
    ms_step = elapsed * 1e3 / args.steps
    dec_avg = float(np.mean(dec_ms))
    log(f"[bench] {args.steps} steps: {ms_step:.4f} ms/step; pa_decode avg {dec_avg:.4f} ms "
        f"(p10 {np.percentile(dec_ms, 10):.4f}, p90 {np.percentile(dec_ms, 90):.4f})")

    if args.copy_calibration:
        copy_calibration(dev)

    comparison = None
    if args.compare_contiguous:
        comparison = compare_contiguous(wl, run, replicas, ws, args, stream)

    gbps = kv_bytes / (ms_step * 1e-3) / 1e9
    achieved = alg_bytes / (dec_avg * 1e-3) / 1e9
    traffic = measured_traffic(args.workload)
    result = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "description": desc, "batch": wl.num_seqs,
                   "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads,
                   "head_dim": wl.head_dim, "block_size": wl.block_size, "kv_dtype": wl.dtype,
                   "out_dtype": "f32", "ctx_mean": round(float(np.mean(ctx)), 1),
                   "ctx_max": int(max(ctx)), "kv_bytes_per_step": kv_bytes,
                   "cache_replicas": len(replicas), "parallelism": "single GPU"},
        "pct_of_peak": round(100 * gbps / PEAK_HBM_GBPS, 2),
        "seqs_per_s": round(wl.num_seqs / (ms_step * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic, "kernel": "pa_decode (partition + combine launches)",
                     "avg_launch_ms": round(dec_avg, 5), "bytes_per_launch": alg_bytes,
                     "launch_ms_p10_median_p90": [round(float(np.percentile(dec_ms, q)), 5) for q in (10, 50, 90)]},
        "cpu_baseline": None,
    }
    if comparison is not None:
        result["paged_vs_contiguous"] = comparison
    if not args.no_prefill:
        result["prefill"] = bench_prefill(args.prefill_steps, args.prefill_warmup, dev, not args.no_cpu_baseline)
        result["prefix_cache"] = bench_prefix(dev, not args.no_cpu_baseline)
        result["swap"] = bench_swap(dev, not args.no_cpu_baseline)
        result["fp8"] = bench_fp8(wl, run, args.workload, dev, args.steps, args.warmup, args.replicas,
                                  not args.no_cpu_baseline, bf16_decode_ms=dec_avg)
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on a CPU sample ...")
        result["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
