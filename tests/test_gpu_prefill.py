"""pa_prefill (chunked causal prefill over the paged cache) against the
float64 oracle.

The cache is built as a serving loop would (prefix admitted, then the chunk
appended with pa_write_kv); the chunk rows' queries come from the workload.
Chunks cross the kernel's 16-row wave tiles and its 4-wave workgroups, and
contexts end inside and at the end of blocks.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_147_amd as P
import workloads as W
from oracle import prefill as PF
from tests._native import NativeDeviceRun, device_tensor
from tests._replay import OracleRun
from tests._tol import assert_close

pytestmark = pytest.mark.gpu


def oracle_rows(wl, rows=None):
    run = OracleRun(wl)
    tables, lens = run.tables(wl)
    return PF.paged_prefill(wl.info["q_rows"], run.cache.k, run.cache.v, tables, lens, wl.info["q_start"],
                            wl.block_size, wl.scale, wl.dtype, wl.num_q_heads, wl.num_kv_heads, rows=rows)


class PrefillRun:
    def __init__(self, wl):
        self.wl = wl
        self.dev = NativeDeviceRun(wl)
        self.q = device_tensor(wl.info["q_rows"], wl.dtype, "cuda")
        self.q_start = torch.from_numpy(wl.info["q_start"].astype(np.int32)).cuda()
        self.max_chunk = int(max(wl.info["chunk"]))

    def run(self, out_dtype=torch.float32, ctx=None):
        wl, dev = self.wl, self.dev
        out = torch.full((self.q.shape[0], wl.num_q_heads, wl.head_dim), float("nan"), dtype=out_dtype,
                         device="cuda")
        P.pa_prefill(out, self.q, dev.k_cache, dev.v_cache, dev.tables, dev.ctx if ctx is None else ctx,
                     self.q_start, wl.scale, self.max_chunk)
        return out


# prefixes and chunks: empty prefix, a one-token chunk, chunks that end inside
# a wave tile, span several 4-wave workgroups, and start mid-block
PREFIX = [0, 17, 100, 300, 5, 64]
CHUNK = [70, 1, 33, 200, 16, 129]

SHAPES = [(dt, d, G, B) for dt in ("f16", "bf16") for d in (64, 128) for G in (1, 2, 4, 8) for B in (8, 16, 32)]


@pytest.mark.parametrize("dtype,d,G,B", SHAPES, ids=str)
def test_prefill_shapes_against_oracle(dtype, d, G, B):
    cap = 512
    wl = W.prefill_chunks(f"pf_{dtype}_{d}_{G}_{B}", PREFIX, CHUNK, (2 * G, 2, d, B, dtype),
                          num_blocks=2 * len(PREFIX) * cap // B, max_blocks=cap // B,
                          seed=SHAPES.index((dtype, d, G, B)))
    print(f"[prefill] {wl.name}", flush=True)
    run = PrefillRun(wl)
    got = run.run().cpu().numpy()
    assert_close(got, oracle_rows(wl), dtype, wl.name)


# float32 accumulation error of an O(1) output (~1e-7 absolute); near zero,
# where the 16-bit spacing is finer (f16 subnormals: 6e-8), it can move the
# rounded result by more than one step, so the check allows this floor too.
F32_FLOOR = 2.5e-7


def ulp(x, dtype):
    """Spacing of the 16-bit output type at |x| (subnormal spacing near 0)."""
    mant, emin = (10, -14) if dtype == "f16" else (7, -126)
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** emin)))
    return 2.0 ** (e - mant)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prefill_native_dtype_output_within_one_step_of_the_probability_bound(dtype):
    wl = W.prefill_chunks("pf_nat", PREFIX, CHUNK, (8, 2, 128, 16, dtype), 192, 32, seed=7)
    run = PrefillRun(wl)
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    got = run.run(out_dtype=tdt).double().cpu().numpy()
    ref = torch.from_numpy(oracle_rows(wl)).to(tdt).double().numpy()
    # The p.V product takes P rounded once to f16 (a bf16 cache's V rows are
    # turned into f16 first, exactly, as every value here is inside the f16
    # range): |dP| <= 2^-11 P.  The output, a P-weighted mean of V rows, then
    # moves by at most 2^-11 max|V|, on top of its own final rounding.
    from oracle.bits import to_f64
    rel = 2.0 ** -11
    bound = rel * np.abs(to_f64(wl.v_rows, dtype)).max()
    tol = np.maximum(ulp(ref, dtype), ulp(got, dtype)) + max(F32_FLOOR, bound)
    bad = np.abs(got - ref) > tol
    if bad.any():
        ref64 = oracle_rows(wl)
        idx = np.argwhere(bad)[:8]
        for i in idx:
            t = tuple(i)
            print("row", t, "got", got[t], "ref_rounded", ref[t], "oracle", ref64[t], "ulp", tol[t], flush=True)
        print("count", int(bad.sum()), "of", bad.size, flush=True)
    assert not bad.any()


def test_prefill_bf16_values_beyond_the_f16_range():
    # A bf16 cache's V rows go into p.V as f16; a pair of steps whose rows
    # hold a value beyond the f16 range sends its workgroup back to the start
    # on bf16 rows with P in two bf16 parts.  Here KV head 0 of sequence 3
    # gets rows around token 200 scaled by 2^17 (so the restart happens after
    # several f16 pairs); its chunk rows that see them take the bf16 path,
    # every other workgroup stays on f16.  Both are checked against the
    # oracle, the scaled rows relative to their largest |V|.
    wl = W.prefill_chunks("pf_wide", PREFIX, CHUNK, (8, 2, 128, 16, "bf16"), 2 * 6 * 512 // 16, 512 // 16, seed=11)
    r0 = next(op[3] for op in wl.setup_ops if op[0] == "alloc" and op[1] == 3)    # sequence 3's prefix rows
    rows = np.arange(r0 + 196, r0 + 214)
    v = wl.v_rows[rows, 0]                                # KV head 0, bf16 bits
    exp = (v >> 7) & 0xFF
    ok = (exp > 0) & (exp < 200)
    v[ok] = v[ok] + np.uint16(17 << 7)                    # times 2^17, exactly
    wl.v_rows[rows, 0] = v
    from oracle.bits import to_f64
    assert np.abs(to_f64(wl.v_rows, "bf16")).max() > 65504
    run = PrefillRun(wl)
    got = run.run().cpu().numpy()
    ref = oracle_rows(wl)
    G = wl.num_q_heads // wl.num_kv_heads
    qs = wl.info["q_start"]
    wide = np.zeros(got.shape[:2], dtype=bool)
    wide[qs[3]:qs[4], :G] = True                          # sequence 3's rows, query heads of KV head 0
    big = np.abs(to_f64(wl.v_rows[:, 0], "bf16")).max()
    assert_close(got[wide] / big, ref[wide] / big, "bf16", "rows over V beyond the f16 range")
    assert_close(got[~wide], ref[~wide], "bf16", "every other row")
    assert np.abs(ref[wide]).max() > 1000                 # the scaled rows did reach the outputs


# contexts whose workgroups walk 1, 2, ..., 9 steps of 32 keys: the ring runs
# its steps in pairs and two pairs per turn, so every remainder of the step
# count (a lone last step, a lone last pair) is met
TURN_PREFIX = [32 * k for k in range(9)]
TURN_CHUNK = [8] * 9


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prefill_every_ring_turn_length(dtype):
    wl = W.prefill_chunks(f"pf_turns_{dtype}", TURN_PREFIX, TURN_CHUNK, (8, 2, 128, 16, dtype), 2 * 9 * 288 // 16,
                          288 // 16, seed=21)
    assert [(c - 1) // 32 + 1 for c in wl.info["ctx"]] == list(range(1, 10))
    print(f"[prefill] {wl.name}", flush=True)
    got = PrefillRun(wl).run().cpu().numpy()
    assert_close(got, oracle_rows(wl), dtype, wl.name)


def test_prefill_every_ring_turn_length_on_the_bf16_fallback():
    # every V row of KV head 0 scaled by 2^17 (beyond the f16 range): each of
    # its workgroups reruns its 1..9 steps on bf16 rows with P split, while
    # KV head 1 stays on the f16 path
    wl = W.prefill_chunks("pf_turns_wide", TURN_PREFIX, TURN_CHUNK, (8, 2, 128, 16, "bf16"), 2 * 9 * 288 // 16,
                          288 // 16, seed=22)
    v = wl.v_rows[:, 0]
    exp = (v >> 7) & 0xFF
    ok = (exp > 0) & (exp < 200)
    v[ok] = v[ok] + np.uint16(17 << 7)                    # times 2^17, exactly
    wl.v_rows[:, 0] = v
    from oracle.bits import to_f64
    big = np.abs(to_f64(wl.v_rows[:, 0], "bf16")).max()
    assert big > 65504
    got = PrefillRun(wl).run().cpu().numpy()
    ref = oracle_rows(wl)
    G = wl.num_q_heads // wl.num_kv_heads
    assert_close(got[:, :G] / big, ref[:, :G] / big, "bf16", "KV head 0 (bf16 fallback)")
    assert_close(got[:, G:], ref[:, G:], "bf16", "KV head 1 (f16 path)")
    assert np.abs(ref[:, :G]).max() > 1000


def test_prefill_one_row_chunks_match_decode():
    # one-token chunks are decode steps: pa_prefill and pa_decode agree
    wl = W.prefill_chunks("pf_dec", [5, 0, 70, 33, 400], [1] * 5, (32, 8, 128, 16, "bf16"), 256, 32, seed=3)
    run = PrefillRun(wl)
    got = run.run()
    dec = torch.empty_like(got)
    P.pa_decode(dec, run.q, run.dev.k_cache, run.dev.v_cache, run.dev.tables, run.dev.ctx, wl.scale)
    assert_close(got.cpu().numpy(), dec.cpu().numpy(), "bf16", "prefill vs decode")
    assert_close(got.cpu().numpy(), oracle_rows(wl), "bf16", "one-row chunks")


def test_prefill_zero_context_rows_and_determinism():
    wl = W.prefill_chunks("pf_zero", PREFIX, CHUNK, (8, 2, 64, 16, "f16"), 192, 32, seed=2)
    run = PrefillRun(wl)
    a = run.run()
    assert torch.equal(a, run.run())                     # run to run: same bits
    ctx = run.dev.ctx.clone()
    ctx[1] = 0
    ctx[3] = -4
    out = run.run(ctx=ctx)
    qs = wl.info["q_start"]
    for s in (1, 3):
        assert torch.count_nonzero(out[qs[s]:qs[s + 1]]) == 0
    keep = [s for s in range(len(PREFIX)) if s not in (1, 3)]
    for s in keep:
        assert torch.equal(out[qs[s]:qs[s + 1]], a[qs[s]:qs[s + 1]])


def test_full_size_prefill_sampled():
    # the Llama-3.1-8B GQA prefill workload (16 sequences, 512-token chunks
    # over cached prefixes of up to 2048 tokens); 64 rows checked one by one
    wl = W.llama31_8b_prefill()
    print(f"[prefill] {wl.name} full size", flush=True)
    run = PrefillRun(wl)
    got = run.run().cpu().numpy()
    rng = np.random.default_rng(5)
    T = got.shape[0]
    pairs = [(int(r), int(h)) for r, h in zip(rng.integers(0, T, 64), rng.integers(0, wl.num_q_heads, 64))]
    pairs += [(0, 0), (T - 1, wl.num_q_heads - 1)]
    ref = oracle_rows(wl, rows=pairs)
    idx = tuple(np.array(pairs).T)
    assert_close(got[idx], ref[idx], wl.dtype, wl.name)
    assert np.isfinite(got).all()
