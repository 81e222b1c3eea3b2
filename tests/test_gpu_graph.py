"""The hot path under HIP graph capture.

A serving loop captures a decode step once and replays it.  The library's
calls only launch kernels on the caller's stream (no allocation, no memset,
no synchronisation when the workspace is passed in), so a captured step must
replay to the same bits as the eager step.  Each graph is replayed several
times with other eager work and synchronisations between replays, and every
replay is compared with the eager result.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_147_amd as P
import workloads as W
from paged_kv_cache_147_amd import _lib as L
from tests._native import NativeDeviceRun, device_tensor

pytestmark = pytest.mark.gpu


def replay_and_check(graph, out, want, reps=4):
    for i in range(reps):
        out.fill_(float("nan"))                   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {i}"


def decode_step_graph(run, wl, kc, vc, step, **kw):
    out = torch.empty((wl.num_seqs, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
    ctx = run.ctx_host.tolist()
    probe = L.decode_args(out, run.q, kc, vc, run.tables, run.ctx, wl.scale, max_ctx=max(ctx), **kw)
    ws = L.workspace_for(P.pa_decode_workspace_bytes(probe), "cuda")

    def call():
        step()
        P.pa_decode(out, run.q, kc, vc, run.tables, run.ctx, wl.scale, max_ctx=max(ctx), workspace=ws, **kw)

    call()                                        # eager
    torch.cuda.synchronize()
    want = out.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.synchronize()
    return g, out, want


def test_decode_step_replays_bitwise():
    wl = W.shared_prefix("graph_sp", 3, 4, 200, [1, 7, 9, 16, 300, 2, 5, 8, 11, 3, 40, 12],
                         (32, 8, 128, 16, "bf16"), 512, 64, seed=8)
    run = NativeDeviceRun(wl)
    rows = torch.cat([torch.arange(r0, r0 + n) for (_, r0, n) in run.step_writes]).cuda()
    slots = torch.cat([sl for (sl, _, _) in run.step_writes])
    k_new = run.k_rows.index_select(0, rows).contiguous()
    v_new = run.v_rows.index_select(0, rows).contiguous()
    step = lambda: P.pa_write_kv(run.k_cache, run.v_cache, k_new, v_new, slots)
    for part in (0, 64):
        g, out, want = decode_step_graph(run, wl, run.k_cache, run.v_cache, step, partition_size=part)
        assert torch.isfinite(want).all()
        replay_and_check(g, out, want)


def test_fp8_decode_step_replays_bitwise():
    wl = W.independent("graph_fp8", [1, 33, 600, 77, 1024], (16, 4, 128, 16, "bf16"), 512, 64, seed=5)
    run = NativeDeviceRun(wl)
    nb, hkv, B, d = run.k_cache.shape
    kc = torch.empty((nb, hkv, B, d), dtype=torch.uint8, device="cuda")
    vc = torch.empty_like(kc)
    flat = lambda c: c.permute(0, 2, 1, 3).reshape(nb * B, hkv, d).contiguous()
    P.pa_write_kv_fp8(kc, vc, flat(run.k_cache), flat(run.v_cache),
                      torch.arange(nb * B, dtype=torch.int64, device="cuda"), 1 / 56, 1 / 72)
    rows = torch.cat([torch.arange(r0, r0 + n) for (_, r0, n) in run.step_writes]).cuda()
    slots = torch.cat([sl for (sl, _, _) in run.step_writes])
    k_new = run.k_rows.index_select(0, rows).contiguous()
    v_new = run.v_rows.index_select(0, rows).contiguous()
    step = lambda: P.pa_write_kv_fp8(kc, vc, k_new, v_new, slots, 1 / 56, 1 / 72)
    g, out, want = decode_step_graph(run, wl, kc, vc, step, k_scale=1 / 56, v_scale=1 / 72)
    assert torch.isfinite(want).all()
    replay_and_check(g, out, want)


def test_prefill_replays_bitwise():
    wl = W.PREFILL_CONFIGS["prefill_small"]()
    run = NativeDeviceRun(wl)
    q = device_tensor(wl.info["q_rows"], wl.dtype, "cuda")
    qs = torch.from_numpy(np.asarray(wl.info["q_start"], dtype=np.int32)).cuda()
    mc = int(max(wl.info["chunk"]))
    out = torch.empty((q.shape[0], wl.num_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
    call = lambda: P.pa_prefill(out, q, run.k_cache, run.v_cache, run.tables, run.ctx, qs, wl.scale, mc)
    call()
    torch.cuda.synchronize()
    want = out.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.synchronize()
    replay_and_check(g, out, want)
