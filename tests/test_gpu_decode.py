"""pa_decode / pa_decode_contiguous against the float64 oracle.

Small cases span several partitions and a ragged tail; every shape family of
the supported set is covered (dtype x head_dim x group x block size).  Also:
native-dtype outputs, bitwise invariances, determinism, edge cases.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_147_amd as P
import workloads as W
from oracle import attention as A
from oracle.bits import to_f64
from tests._native import NativeDeviceRun, device_tensor
from tests._replay import OracleRun, contiguous_layout
from tests._tol import assert_close, errors

pytestmark = pytest.mark.gpu


def oracle_out(wl, heads=None):
    run = OracleRun(wl)
    tables, lens = run.tables(wl)
    return A.paged_decode(wl.q, run.cache.k, run.cache.v, tables, lens, wl.block_size, wl.scale,
                          wl.dtype, wl.num_q_heads, wl.num_kv_heads, heads=heads)


def ragged(S, seed, lo=1, hi=700):
    rng = np.random.default_rng(seed)
    ctx = rng.integers(lo, hi, size=S).tolist()
    ctx[0] = lo            # shortest
    ctx[-1] = hi           # longest
    return ctx


SHAPES = []
for dtype in ("f32", "f16", "bf16"):
    for d in (64, 128):
        for G in (1, 2, 4, 8):
            for B in (8, 16, 32):
                SHAPES.append((dtype, d, G, B))


@pytest.mark.parametrize("dtype,d,G,B", SHAPES, ids=lambda x: str(x))
def test_shapes_against_oracle(dtype, d, G, B):
    hkv = 2
    ctx = ragged(5, seed=d + G + B, hi=600)
    cap = 640
    wl = W.independent(f"shape_{dtype}_{d}_{G}_{B}", ctx, (G * hkv, hkv, d, B, dtype),
                       num_blocks=2 * sum(cap // B for _ in ctx), max_blocks=cap // B,
                       seed=SHAPES.index((dtype, d, G, B)))
    print(f"[decode] {wl.name} ctx={ctx}", flush=True)
    dev = NativeDeviceRun(wl)
    ref = oracle_out(wl)
    for part in (0, 64, 512):
        got = dev.decode(partition_size=part).cpu().numpy()
        assert_close(got, ref, dtype, f"{wl.name} partition {part}")


@pytest.mark.parametrize("name,make", [
    ("tiny", lambda: W.tiny()),
    ("shared_prefix", lambda: W.shared_prefix("sp", 3, 4, 1008, [1, 7, 9, 16, 300, 2, 5, 8, 11, 3, 400, 12],
                                              (32, 8, 128, 16, "bf16"), 1024, 512, seed=8)),
    ("beam", lambda: W.beam_fork("bm", 2, 4, 4095, (8, 8, 128, 16, "f16"), 1200, 256, seed=6)),
])
def test_workloads_against_oracle(name, make):
    wl = make()
    print(f"[decode] {name}", flush=True)
    dev = NativeDeviceRun(wl)
    ref = oracle_out(wl)
    assert_close(dev.decode().cpu().numpy(), ref, wl.dtype, name)


# float32 accumulation error of an O(1) output (~1e-7 absolute); near zero,
# where the 16-bit spacing is finer (f16 subnormals: 6e-8), it can move the
# rounded result by more than one step, so the check allows this floor too.
F32_FLOOR = 2.5e-7


def ulp(x, dtype):
    """Spacing of the 16-bit output type at |x| (subnormal spacing near 0)."""
    mant, emin = (10, -14) if dtype == "f16" else (7, -126)
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** emin)))
    return 2.0 ** (e - mant)


def record_round_bound(wl):
    """What the split-context records add: a context of several partitions is
    merged from records whose weighted sums o_p are stored in f16 under a
    power-of-two scale (each value within 2^-11 of itself); the merge divides
    sum_p w_p o_p by sum_p w_p l_p with |o_p| <= l_p max|V|, so an output moves
    by at most 2^-11 max|V|."""
    vmax = float(np.max(np.abs(to_f64(wl.v_rows, wl.dtype)))) if wl.v_rows.size else 0.0
    return 2.0 ** -11 * vmax


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_native_dtype_output_within_one_ulp(dtype):
    # within one spacing of the output type of the oracle rounded once, plus
    # the records' bound where a context spans several partitions
    wl = W.independent("nat", ragged(6, 1, hi=900), (8, 2, 128, 16, dtype), 600, 64, seed=2)
    dev = NativeDeviceRun(wl)
    ref = oracle_out(wl)
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    ref_r = torch.from_numpy(ref).to(tdt).double().numpy()      # the oracle rounded once
    ctx = np.asarray(wl.info["ctx"])
    for part in (0, 128, 512):
        got = dev.decode(out_dtype=tdt, partition_size=part).double().cpu().numpy()
        eff = part or 128                                        # automatic: at least 128 tokens
        multi = (ctx > eff)[:, None, None]                       # sequences merged from records
        tol = np.maximum(np.maximum(ulp(ref_r, dtype), ulp(got, dtype)), F32_FLOOR)
        tol = tol + np.where(multi, record_round_bound(wl), 0.0)
        assert np.all(np.abs(got - ref_r) <= tol), part


@pytest.mark.parametrize("shift", [100, -100])
def test_records_keep_values_far_from_one(shift):
    # The split-context records of a 16-bit cache hold f16 values under a
    # power-of-two scale per row.  V rows scaled by 2^100 or 2^-100 (exact in
    # bf16, far outside the f16 range) must merge like ordinary ones: no
    # overflow to inf, no flush to zero, the usual error relative to the scale.
    wl = W.independent(f"rec{shift}", [1500, 700, 1300, 40], (8, 2, 128, 16, "bf16"), 400, 128, seed=11)
    v = wl.v_rows
    before = to_f64(v.copy(), "bf16")
    e = ((v >> 7) & 0xFF).astype(np.int32)
    nz = e != 0
    v[nz] = (v[nz] & 0x807F) | ((e[nz] + shift).astype(np.uint16) << 7)   # exponent field + shift
    assert np.array_equal(to_f64(v, "bf16"), before * 2.0 ** shift)
    dev = NativeDeviceRun(wl)
    ref = oracle_out(wl)
    for part in (0, 128):
        got = dev.decode(partition_size=part).cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(got)), part
        assert_close(got / 2.0 ** shift, ref / 2.0 ** shift, "bf16", f"V scaled by 2^{shift}, partition {part}")


def test_relabelling_sharing_and_repeat_are_bitwise_identical():
    mk = lambda share: W.shared_prefix("sp", 2, 4, 1008, [1, 7, 9, 300, 2, 5, 400, 12],
                                       (16, 4, 128, 16, "bf16"), 1024, 512, share=share, seed=8)
    a = NativeDeviceRun(mk(True))
    other = np.random.default_rng(5).permutation(1024).astype(np.int32)
    b = NativeDeviceRun(mk(True), free_order=other)
    c = NativeDeviceRun(mk(False))
    assert not torch.equal(a.tables, b.tables)
    oa, ob, oc = a.decode(), b.decode(), c.decode()
    assert torch.equal(oa, ob) and torch.equal(oa, oc)
    assert torch.equal(oa, a.decode())        # run-to-run determinism


def test_contiguous_kernel_matches_oracle_and_paged_bitwise():
    for B in (8, 16, 32):
        wl = W.block_sweep(B, batch=6, ctx=1000)
        dev = NativeDeviceRun(wl)
        k, v, ctx = contiguous_layout(wl, capacity=1024)
        kd, vd = device_tensor(k, wl.dtype, "cuda"), device_tensor(v, wl.dtype, "cuda")
        out = torch.empty((wl.num_seqs, wl.num_q_heads, wl.head_dim), device="cuda")
        P.pa_decode_contiguous(out, dev.q, kd, vd, torch.from_numpy(ctx).cuda(), wl.scale)
        paged = dev.decode()
        # same score path (matrix cores; at B = 8 a tile's halves come from two
        # blocks), same order of every sum: bit-identical
        assert torch.equal(out, paged), B
        ref = A.contiguous_decode(wl.q, k, v, ctx, wl.scale, wl.dtype, wl.num_q_heads, wl.num_kv_heads)
        assert_close(out.cpu().numpy(), ref, wl.dtype, f"contiguous B={B}")
        assert_close(paged.cpu().numpy(), ref, wl.dtype, f"paged B={B}")


@pytest.mark.parametrize("part", [8, 24, 40, 136])
def test_contiguous_odd_partitions(part):
    # partitions that are multiples of 8 but not of 16: score tiles start mid-way
    wl = W.independent("codd", [1, 9, 23, 100, 333], (8, 2, 128, 8, "bf16"), 256, 48, seed=31)
    k, v, ctx = contiguous_layout(wl, capacity=344)
    kd, vd = device_tensor(k, wl.dtype, "cuda"), device_tensor(v, wl.dtype, "cuda")
    q = device_tensor(wl.q, wl.dtype, "cuda")
    out = torch.empty((wl.num_seqs, wl.num_q_heads, wl.head_dim), device="cuda")
    P.pa_decode_contiguous(out, q, kd, vd, torch.from_numpy(ctx).cuda(), wl.scale, partition_size=part)
    ref = A.contiguous_decode(wl.q, k, v, ctx, wl.scale, wl.dtype, wl.num_q_heads, wl.num_kv_heads)
    assert_close(out.cpu().numpy(), ref, wl.dtype, f"contiguous partition {part}")


@pytest.mark.parametrize("dtype,G", [("bf16", 4), ("f32", 1)])
def test_more_than_64_partition_records(dtype, G):
    # 8-token partitions: up to 138 records per (sequence, head), so the merge
    # runs several rounds of 64 records and several batches in each
    ctx = [1, 9, 64, 520, 1100]
    wl = W.independent(f"many_{dtype}", ctx, (2 * G, 2, 64, 8, dtype), 512, 140, seed=17)
    dev = NativeDeviceRun(wl)
    ref = oracle_out(wl)
    for part in (8, 16):
        assert_close(dev.decode(partition_size=part).cpu().numpy(), ref, dtype, f"{wl.name} partition {part}")


def test_edge_contexts():
    # ctx 1, 7, 8, 9, exactly one and two partitions, the table's maximum
    ctx = [1, 7, 8, 9, 256, 257, 512, 1024]
    wl = W.independent("edge", ctx, (8, 2, 128, 16, "bf16"), 256, 64, seed=11)
    dev = NativeDeviceRun(wl)
    ref = oracle_out(wl)
    assert_close(dev.decode().cpu().numpy(), ref, "bf16", "edge")
    # ctx 1 gives the single V row, widened exactly
    one = dev.decode().cpu().numpy()[0]
    vrow = dev.v_rows[wl.step_ops[0][3]].float().cpu().numpy()     # seq 0's only token
    assert np.array_equal(one.reshape(2, 4, 128)[:, 0, :], vrow)


def test_longest_contexts_and_widest_batch():
    # contexts of 32768 and 16384 tokens (128 and 64 records per (sequence,
    # head): the automatic choice here is 256-token partitions) next to a
    # 3-token one; then 2048 short sequences (a wide grid of single-partition
    # units)
    wl = W.independent("long32k", [32768, 16384, 3], (32, 8, 128, 16, "bf16"), 3200, 2048, seed=31)
    print(f"[decode] {wl.name}", flush=True)
    dev = NativeDeviceRun(wl)
    ref = oracle_out(wl)
    assert_close(dev.decode().cpu().numpy(), ref, "bf16", wl.name)
    assert_close(dev.decode(partition_size=128).cpu().numpy(), ref, "bf16", wl.name + " 128-token partitions")
    ctx = np.random.default_rng(33).integers(1, 65, 2048)
    wl = W.independent("wide2k", ctx.tolist(), (32, 8, 128, 16, "bf16"), 2048 * 4, 4, seed=34)
    print(f"[decode] {wl.name}", flush=True)
    dev = NativeDeviceRun(wl)
    assert_close(dev.decode().cpu().numpy(), oracle_out(wl), "bf16", wl.name)


def test_zero_and_negative_context_give_zero_rows():
    wl = W.independent("z", [5, 40], (8, 2, 64, 16, "f16"), 64, 8, seed=1)
    dev = NativeDeviceRun(wl)
    ctx = torch.tensor([0, -3], dtype=torch.int32, device="cuda")
    out = dev.decode(ctx=ctx)
    assert torch.count_nonzero(out) == 0


def test_unwritten_slots_never_leak():
    # every never-written slot holds NaN; a finite output proves none was used
    wl = W.independent("nan", [3, 17, 33, 250], (8, 8, 128, 32, "bf16"), 64, 8, seed=4)
    dev = NativeDeviceRun(wl)
    k, _ = dev.cache_bits()
    assert (k == 0x7FC0).sum() > 0
    assert torch.isfinite(dev.decode(partition_size=64)).all()


def test_workspace_reuse_across_calls():
    # one workspace serves successive calls with different contexts
    wl = W.independent("reuse", [1, 100, 300, 700, 1500, 33], (8, 2, 128, 16, "bf16"), 700, 96, seed=21)
    dev = NativeDeviceRun(wl)
    ref = oracle_out(wl)
    out = torch.empty((wl.num_seqs, wl.num_q_heads, wl.head_dim), device="cuda")
    ws = None
    firsts = []
    for rep in range(3):
        ws = P.pa_decode(out, dev.q, dev.k_cache, dev.v_cache, dev.tables, dev.ctx, wl.scale,
                         partition_size=64, workspace=ws)
        firsts.append(out.clone())
        # a shorter batch in between, on the same workspace
        short = torch.clamp(dev.ctx - 50, min=1)
        P.pa_decode(out, dev.q, dev.k_cache, dev.v_cache, dev.tables, short, wl.scale,
                    partition_size=64, workspace=ws)
    assert all(torch.equal(firsts[0], f) for f in firsts[1:])
    assert_close(firsts[0].cpu().numpy(), ref, "bf16", "reuse")


# ---- empty contexts between long ones ------------------------------------------

LONG_CTX = [1, 2000, 37, 449, 896, 1500, 17, 912]


@pytest.mark.parametrize("part", [0, 64, 512])
def test_mixed_empty_and_long_contexts(part):
    # empty and negative contexts between real ones: zero rows; the others
    # span one to 32 partitions
    wl = W.independent("mixed_empty", LONG_CTX, (8, 2, 128, 16, "bf16"), 2048, 128, seed=3)
    dev = NativeDeviceRun(wl)
    lens = np.array([1, 0, 37, -3, 896, 0, 17, 911], dtype=np.int32)   # within each sequence's tokens
    run = OracleRun(wl)
    tables, _ = run.tables(wl)
    live = [(s, h) for s in range(wl.num_seqs) if lens[s] > 0 for h in range(wl.num_q_heads)]
    ref = A.paged_decode(wl.q, run.cache.k, run.cache.v, tables, np.maximum(lens, 0), wl.block_size,
                         wl.scale, wl.dtype, wl.num_q_heads, wl.num_kv_heads, heads=live)
    got = dev.decode(ctx=torch.from_numpy(lens).cuda(), partition_size=part).cpu().numpy()
    assert np.all(got[lens <= 0] == 0)
    assert_close(got, ref, "bf16", f"empty contexts, partition {part}")


@pytest.mark.parametrize("share", [True, False], ids=["shared_prefix", "no_share"])
def test_full_size_gqa_sampled(share):
    # the benchmarked workload (Llama-3.1-8B layer, 256 sequences) in the
    # benchmarked launch (automatic fixed partitions) and in 128-token
    # partitions; 50 (sequence, head) rows checked against the oracle one by one
    wl = W.llama31_8b_gqa(share=share)
    print(f"[decode] {wl.name} full size", flush=True)
    dev = NativeDeviceRun(wl)
    got = dev.decode().cpu().numpy()
    p128 = dev.decode(partition_size=128).cpu().numpy()
    rng = np.random.default_rng(11)
    pairs = [(int(s), int(h)) for s, h in zip(rng.integers(0, wl.num_seqs, 48), rng.integers(0, wl.num_q_heads, 48))]
    pairs += [(0, 0), (wl.num_seqs - 1, wl.num_q_heads - 1)]
    ref = oracle_out(wl, heads=pairs)
    idx = tuple(np.array(pairs).T)
    assert_close(got[idx], ref[idx], wl.dtype, wl.name)
    assert_close(p128[idx], ref[idx], wl.dtype, wl.name + " 128-token partitions")
    assert np.isfinite(got).all() and np.isfinite(p128).all()


# ---- debug validation --------------------------------------------------------

def test_validate_counts_bad_tables_and_lengths():
    wl = W.independent("val", [5, 40, 300, 17], (8, 2, 64, 16, "f16"), 128, 32, seed=9)
    dev = NativeDeviceRun(wl)
    assert P.pa_decode_validate(dev.q, dev.k_cache, dev.v_cache, dev.tables, dev.ctx) == 0
    tables = dev.tables.clone()
    tables[1, 0] = -5                      # read block of seq 1
    tables[2, 18] = wl.num_blocks + 3      # read block of seq 2 (ctx 300 -> 19 blocks)
    tables[0, 5] = -7                      # padding past ceil(5 / 16): never read, not counted
    ctx = dev.ctx.clone()
    ctx[3] = 32 * 16 + 1                   # above the table's capacity: counted once, and the
    #                                        clamped 512 tokens would read 30 padding entries (-1)
    assert P.pa_decode_validate(dev.q, dev.k_cache, dev.v_cache, tables, dev.ctx) == 2
    assert P.pa_decode_validate(dev.q, dev.k_cache, dev.v_cache, dev.tables, ctx) == 1 + 30
    assert P.pa_decode_validate(dev.q, dev.k_cache, dev.v_cache, tables, ctx) == 2 + 1 + 30


def test_validate_on_another_stream():
    # the count is allocated on the current stream and filled on the caller's:
    # the binding orders the two, so the count read back is the check's
    wl = W.independent("val_stream", [5, 40, 300, 17], (8, 2, 64, 16, "f16"), 128, 32, seed=9)
    dev = NativeDeviceRun(wl)
    tables = dev.tables.clone()
    tables[1, 0] = -5
    tables[2, 18] = wl.num_blocks + 3
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        st = P.current_stream()
    for _ in range(3):
        assert P.pa_decode_validate(dev.q, dev.k_cache, dev.v_cache, tables, dev.ctx, stream=st) == 2
        assert P.pa_decode_validate(dev.q, dev.k_cache, dev.v_cache, dev.tables, dev.ctx, stream=st) == 0


def test_debug_env_rejects_bad_tables_before_decoding():
    # PAGEDKV_DEBUG is read once per process: run the check in a child
    import os
    import subprocess
    import sys
    code = r"""
import torch, workloads as W, paged_kv_cache_147_amd as P
from tests._native import NativeDeviceRun
wl = W.independent("dbg", [5, 40, 300, 17], (8, 2, 64, 16, "f16"), 128, 32, seed=9)
dev = NativeDeviceRun(wl)
out = torch.full((wl.num_seqs, wl.num_q_heads, wl.head_dim), 7.0, device="cuda")
P.pa_decode(out, dev.q, dev.k_cache, dev.v_cache, dev.tables, dev.ctx, wl.scale)
ok = bool(torch.isfinite(out).all())
bad = dev.tables.clone(); bad[2, 3] = -1
out.fill_(7.0)
try:
    P.pa_decode(out, dev.q, dev.k_cache, dev.v_cache, bad, dev.ctx, wl.scale)
    print("NO_ERROR")
except P.PagedKVError as e:
    print("REJECTED", ok, bool((out == 7.0).all()), str(e)[:80])
"""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, PAGEDKV_DEBUG="1")
    r = subprocess.run([sys.executable, "-c", code], cwd=root, env=env, capture_output=True, text=True, timeout=100)
    print(r.stdout[-500:], r.stderr[-500:], flush=True)
    assert r.returncode == 0
    assert "REJECTED True True" in r.stdout          # good call ran; bad call launched nothing


def test_workspace_made_by_the_binding_on_any_stream():
    # with no workspace the binding allocates one; it must work on the default
    # stream (handle 0) and on another stream (which first waits for the
    # current stream's queued work, and the allocator is told the memory is in
    # use there)
    wl = W.independent("ws_streams", [5, 700, 1300], (8, 2, 128, 16, "bf16"), 256, 96, seed=12)
    dev = NativeDeviceRun(wl)
    ref = oracle_out(wl)
    want = dev.decode(partition_size=128)
    for use_side in (False, True):
        out = torch.empty_like(want)
        side = torch.cuda.Stream()
        if use_side:
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                st = P.current_stream()
            P.pa_decode(out, dev.q, dev.k_cache, dev.v_cache, dev.tables, dev.ctx, wl.scale, partition_size=128,
                        stream=st)
            torch.cuda.current_stream().wait_stream(side)
        else:
            P.pa_decode(out, dev.q, dev.k_cache, dev.v_cache, dev.tables, dev.ctx, wl.scale, partition_size=128,
                        stream=P.current_stream())
        torch.cuda.synchronize()
        assert torch.equal(out, want), use_side
        assert_close(out.cpu().numpy(), ref, wl.dtype, f"side stream {use_side}")
