"""Pins of the float64 prefill oracle (CPU only).

Each pin checks the oracle against something it does not compute itself:
causal scaled-dot-product attention from torch on the workload's own rows
(no block table involved), the decode oracle for one-row chunks, closed
forms of softmax averaging, and a count of the work.  Planted mistakes (a
query that sees one token too few or too many, the wrong KV head) must fail
the first pin.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from oracle import prefill as PF
from oracle.bits import to_f64
from tests._replay import OracleRun, logical_streams


def run_oracle(wl, **kw):
    run = OracleRun(wl)
    tables, lens = run.tables(wl)
    return PF.paged_prefill(wl.info["q_rows"], run.cache.k, run.cache.v, tables, lens,
                            wl.info["q_start"], wl.block_size, wl.scale, wl.dtype,
                            wl.num_q_heads, wl.num_kv_heads, **kw), lens


def sdpa_reference(wl):
    """torch SDPA, float64, on each sequence's K/V rows in token order (taken
    from the workload's row arrays, not from any cache or table), with a
    boolean causal mask aligned to the end of the context."""
    streams = logical_streams(wl)
    G = wl.num_q_heads // wl.num_kv_heads
    qs = wl.info["q_start"]
    out = np.zeros((qs[-1], wl.num_q_heads, wl.head_dim))
    for s in wl.batch:
        rows = streams[s]
        ctx, n = len(rows), qs[s + 1] - qs[s]
        k = torch.from_numpy(to_f64(wl.k_rows[rows], wl.dtype)).permute(1, 0, 2)   # [Hkv][ctx][d]
        v = torch.from_numpy(to_f64(wl.v_rows[rows], wl.dtype)).permute(1, 0, 2)
        k = k.repeat_interleave(G, dim=0).contiguous()
        v = v.repeat_interleave(G, dim=0).contiguous()
        q = torch.from_numpy(to_f64(wl.info["q_rows"][qs[s]:qs[s + 1]], wl.dtype)).permute(1, 0, 2).contiguous()
        pos = torch.arange(ctx - n, ctx)
        mask = torch.arange(ctx)[None, :] <= pos[:, None]                           # [n][ctx]
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=wl.scale)
        out[qs[s]:qs[s + 1]] = o.permute(1, 0, 2).numpy()
    return out


def small(dtype="bf16", G=4, B=16):
    return W.prefill_chunks(f"pf_{dtype}_{G}_{B}", [0, 17, 100, 45], [9, 33, 20, 1],
                            (2 * G, 2, 64, B, dtype), num_blocks=64, max_blocks=16, seed=G + B)


@pytest.mark.parametrize("dtype,G,B", [("bf16", 4, 16), ("f16", 1, 8), ("f32", 2, 32)])
def test_prefill_matches_causal_sdpa(dtype, G, B):
    wl = small(dtype, G, B)
    got, _ = run_oracle(wl)
    ref = sdpa_reference(wl)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_one_row_chunks_equal_decode():
    # a chunk of one token is a decode step of that token
    wl = W.prefill_chunks("pf_dec", [5, 0, 70, 33], [1, 1, 1, 1], (8, 2, 64, 16, "bf16"), 32, 8, seed=3)
    got, lens = run_oracle(wl)
    run = OracleRun(wl)
    tables, _ = run.tables(wl)
    dec = A.paged_decode(wl.info["q_rows"], run.cache.k, run.cache.v, tables, lens, wl.block_size,
                         wl.scale, wl.dtype, wl.num_q_heads, wl.num_kv_heads)
    assert np.array_equal(got, dec)


def test_closed_forms():
    wl = small("f32", 2, 16)
    # constant V rows: every output equals the constant
    c = np.float32(1.75).view(np.uint32)
    wl.v_rows[...] = c
    got, _ = run_oracle(wl)
    assert np.allclose(got, 1.75, atol=1e-15)
    # zero queries: each row is the mean of the V rows it can see
    wl = small("f32", 2, 16)
    wl.info["q_rows"][...] = 0
    got, lens = run_oracle(wl)
    streams = logical_streams(wl)
    qs = wl.info["q_start"]
    for s in wl.batch:
        v = to_f64(wl.v_rows[streams[s]], "f32")                 # [ctx][Hkv][d]
        for r, p in zip(range(qs[s], qs[s + 1]), PF.chunk_positions(lens[s], qs[s + 1] - qs[s])):
            want = v[:p + 1].mean(axis=0)                         # [Hkv][d]
            assert np.allclose(got[r], np.repeat(want, 2, axis=0), atol=1e-12)


def test_rows_subset_matches_full():
    wl = small()
    full, _ = run_oracle(wl)
    pairs = [(0, 0), (5, 7), (40, 3), (62, 1)]
    part, _ = run_oracle(wl, rows=pairs)
    for r, h in pairs:
        assert np.array_equal(part[r, h], full[r, h])
    mask = np.ones(full.shape[:2], bool)
    for r, h in pairs:
        mask[r, h] = False
    assert not np.any(part[mask])


def test_flop_count_closed_form():
    # a whole prompt of n tokens: sum over rows of (p + 1) = n (n + 1) / 2
    n, d, hq = 37, 64, 8
    assert PF.prefill_flops([n], [0, n], d, hq) == n * (n + 1) // 2 * 4 * d * hq
    # a one-row chunk at the end of a 100-token context: 100 visible tokens
    assert PF.prefill_flops([100], [0, 1], d, hq) == 100 * 4 * d * hq


@pytest.mark.parametrize("mutant", ["sees_one_less", "sees_one_more", "wrong_kv_head"])
def test_planted_mistakes_fail_the_sdpa_pin(mutant, monkeypatch):
    wl = small("bf16", 4, 16)
    ref = sdpa_reference(wl)
    if mutant == "sees_one_less":
        monkeypatch.setattr(PF, "chunk_positions", lambda c, n: np.maximum(np.arange(c - n, c) - 1, 0))
    elif mutant == "sees_one_more":
        monkeypatch.setattr(PF, "chunk_positions", lambda c, n: np.minimum(np.arange(c - n, c) + 1, c - 1))
    else:
        # every query reads the other KV head: swap the two heads in the cache
        run = OracleRun(wl)
        tables, lens = run.tables(wl)
        got = PF.paged_prefill(wl.info["q_rows"], run.cache.k[:, ::-1].copy(), run.cache.v[:, ::-1].copy(),
                               tables, lens, wl.info["q_start"], wl.block_size, wl.scale, wl.dtype,
                               wl.num_q_heads, wl.num_kv_heads)
        assert np.max(np.abs(got - ref)) > 1e-3
        return
    got, _ = run_oracle(wl)
    assert np.max(np.abs(got - ref)) > 1e-3
