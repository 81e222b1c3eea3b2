"""pa_swap_out / pa_swap_in (block copies to and from pinned host memory).

Bit copies, so the checks are exact: the host buffer holds the listed blocks
in the documented layout, a round trip into other blocks reproduces them,
invalid ids are skipped, and a decode batch whose sequences are swapped out
(pool + device), their freed blocks overwritten, and swapped back in gives
the same output bits as before (decode results do not depend on which
physical blocks hold the tokens).
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_147_amd as P
import workloads as W
from tests._native import NativeDeviceRun

pytestmark = pytest.mark.gpu


def caches(nb, hkv, B, d, dtype, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    bits = torch.randint(-2 ** 15, 2 ** 15, (2, nb, hkv, B, d), generator=g, dtype=torch.int32).to(torch.int16)
    kv = bits.view(dtype).cuda()
    return kv[0].contiguous(), kv[1].contiguous()


@pytest.mark.parametrize("dtype,hkv,B,d", [(torch.bfloat16, 8, 16, 128), (torch.float16, 2, 8, 64),
                                            (torch.bfloat16, 4, 32, 128)])
def test_swap_out_layout_and_round_trip(dtype, hkv, B, d):
    nb = 48
    k, v = caches(nb, hkv, B, d, dtype, seed=B + hkv)
    blocks = [7, 3, 47, 0, 12, 30]
    n = len(blocks)
    host = torch.zeros((n, 2, hkv, B, d), dtype=dtype).pin_memory()
    P.pa_swap_out(k, v, torch.tensor(blocks, dtype=torch.int32, device="cuda"), host)
    torch.cuda.synchronize()
    kc, vc = k.cpu(), v.cpu()
    for i, b in enumerate(blocks):
        assert torch.equal(host[i, 0].view(torch.int16), kc[b].view(torch.int16))
        assert torch.equal(host[i, 1].view(torch.int16), vc[b].view(torch.int16))
    dest = [20, 21, 22, 23, 24, 25]
    P.pa_swap_in(k, v, torch.tensor(dest, dtype=torch.int32, device="cuda"), host)
    torch.cuda.synchronize()
    k2, v2 = k.cpu(), v.cpu()
    for b_old, b_new in zip(blocks, dest):
        assert torch.equal(k2[b_new].view(torch.int16), kc[b_old].view(torch.int16))
        assert torch.equal(v2[b_new].view(torch.int16), vc[b_old].view(torch.int16))
    untouched = [b for b in range(nb) if b not in dest]
    assert torch.equal(k2[untouched].view(torch.int16), kc[untouched].view(torch.int16))
    assert torch.equal(v2[untouched].view(torch.int16), vc[untouched].view(torch.int16))


def test_invalid_ids_are_skipped():
    nb, hkv, B, d = 16, 2, 16, 64
    k, v = caches(nb, hkv, B, d, torch.float16, seed=3)
    host = torch.full((3, 2, hkv, B, d), 7, dtype=torch.int16).pin_memory().view(torch.float16)
    ids = torch.tensor([-1, 5, nb], dtype=torch.int32, device="cuda")
    P.pa_swap_out(k, v, ids, host)
    torch.cuda.synchronize()
    hv = host.view(torch.int16)
    assert bool((hv[0] == 7).all()) and bool((hv[2] == 7).all())
    assert torch.equal(hv[1, 0], k[5].cpu().view(torch.int16))
    before = (k.cpu().clone(), v.cpu().clone())
    P.pa_swap_in(k, v, ids, host)
    torch.cuda.synchronize()
    assert torch.equal(k.cpu().view(torch.int16)[[b for b in range(nb) if b != 5]],
                       before[0].view(torch.int16)[[b for b in range(nb) if b != 5]])


def test_unpinned_or_short_host_buffers_are_refused():
    k, v = caches(8, 2, 16, 64, torch.float16, seed=1)
    ids = torch.tensor([1, 2], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        P.pa_swap_out(k, v, ids, torch.empty((2, 2, 2, 16, 64), dtype=torch.float16))       # not pinned
    with pytest.raises(ValueError):
        P.pa_swap_out(k, v, ids, torch.empty((1, 2, 2, 16, 64), dtype=torch.float16).pin_memory())  # short


def decode(run, wl, tables, ctx):
    out = torch.empty((wl.num_seqs, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
    P.pa_decode(out, run.q, run.k_cache, run.v_cache, tables, ctx, wl.scale)
    return out


@pytest.mark.parametrize("share", [True, False])
def test_swap_preempts_and_restores_a_decode_batch(share):
    # 6 groups of 4 sequences behind a 100-token prompt (forked when shared)
    lens = np.random.default_rng(5).integers(1, 200, size=24)
    wl = W.shared_prefix("swap_batch", 6, 4, 100, lens, (16, 8, 128, 16, "bf16"), 1024, 32, share=share)
    run = NativeDeviceRun(wl)
    pool = run.pool_run.pool
    ref = decode(run, wl, run.tables, run.ctx)
    victims = [s for s in wl.batch if s % 3 == 1]
    hosts = {}
    for s in victims:
        blocks = pool.swap_out(s)
        host = torch.empty((len(blocks), 2, wl.num_kv_heads, wl.block_size, wl.head_dim),
                           dtype=run.k_cache.dtype).pin_memory()
        P.pa_swap_out(run.k_cache, run.v_cache, torch.from_numpy(blocks).cuda(), host)
        hosts[s] = host
    torch.cuda.synchronize()
    # whatever now reuses the freed blocks overwrites them
    freed = [b for b in range(wl.num_blocks) if pool.refcount(b) == 0]
    fill = torch.full((len(freed), wl.num_kv_heads, wl.block_size, wl.head_dim), 3.0, dtype=run.k_cache.dtype,
                      device="cuda")
    run.k_cache[freed] = fill
    run.v_cache[freed] = fill
    for s in victims:
        blocks = pool.swap_in(s)
        P.pa_swap_in(run.k_cache, run.v_cache, torch.from_numpy(blocks).cuda(), hosts[s])
    torch.cuda.synchronize()
    tables, ctx = pool.block_tables(wl.batch, wl.max_blocks)
    got = decode(run, wl, torch.from_numpy(tables).cuda(), torch.from_numpy(ctx).cuda())
    assert torch.equal(got, ref)
