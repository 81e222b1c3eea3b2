"""Oracle attention pinned to a library routine, closed forms and invariants.

* The paged oracle must equal torch's scaled_dot_product_attention (float64,
  CPU) run on each sequence's logical K/V stream, which is rebuilt from the
  op log without blocks or tables.  The pages hold that paging leaves the
  attention unchanged ("vllm-pagedattention" (chenyuan1125.github.io),
  页表真正解开的…), so this library routine is the expected value.
* Softmax closed forms: one token, zero query, constant V, dominant score.
* Invariants: relabelling physical blocks and sharing prefix blocks change
  nothing, bit for bit ("Paged Attention" (daiw.org), 直觉: any logical ->
  physical mapping is legal; "vllm-pagedattention", 一块内存…: shared
  prefixes point at the same physical blocks).
* The split-context combine gives back the one-pass result.
* Planted mistakes in a copy of the oracle are caught by these pins.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from oracle.bits import to_f64
from tests._replay import OracleRun, logical_streams

SMALL = {
    "tiny_f32": lambda: W.tiny(),
    "gqa4_bf16_b4": lambda: W.independent("g4", [1, 5, 8, 9, 31, 64], (8, 2, 16, 4, "bf16"),
                                          64, 16, seed=3),
    "gqa8_f16_b8": lambda: W.independent("g8", [3, 17, 40], (8, 1, 32, 8, "f16"), 32, 8, seed=4),
    "mha_shared_bf16": lambda: W.shared_prefix("sp", 2, 3, 24, [5, 17, 30, 3, 9, 16],
                                               (4, 4, 16, 8, "bf16"), 64, 16, seed=5),
    "beam_f16": lambda: W.beam_fork("bm", 2, 4, 37, (4, 2, 16, 8, "f16"), 64, 8, seed=6),
}


def sdpa_reference(wl):
    """torch SDPA (float64, CPU) on the logical streams, GQA by h // group."""
    streams = logical_streams(wl)
    group = wl.num_q_heads // wl.num_kv_heads
    out = np.zeros((wl.num_seqs, wl.num_q_heads, wl.head_dim))
    for i, s in enumerate(wl.batch):
        rows = np.asarray(streams[s])
        k = torch.from_numpy(to_f64(wl.k_rows[rows], wl.dtype)).permute(1, 0, 2)
        v = torch.from_numpy(to_f64(wl.v_rows[rows], wl.dtype)).permute(1, 0, 2)
        k = k.repeat_interleave(group, dim=0).contiguous()
        v = v.repeat_interleave(group, dim=0).contiguous()
        q = torch.from_numpy(to_f64(wl.q[i], wl.dtype)).unsqueeze(1)     # [Hq][1][d]
        o = torch.nn.functional.scaled_dot_product_attention(
            q.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0), scale=wl.scale)
        out[i] = o[0, :, 0, :].numpy()
    return out


def run_paged(wl, fn=A.paged_decode, free_order=None):
    run = OracleRun(wl, free_order)
    tables, lens = run.tables(wl)
    return fn(wl.q, run.cache.k, run.cache.v, tables, lens, wl.block_size, wl.scale,
              wl.dtype, wl.num_q_heads, wl.num_kv_heads)


@pytest.mark.parametrize("name", sorted(SMALL))
def test_paged_equals_library_sdpa(name):
    wl = SMALL[name]()
    got = run_paged(wl)
    ref = sdpa_reference(wl)
    assert np.max(np.abs(got - ref)) < 1e-12


@pytest.mark.parametrize("name", sorted(SMALL))
def test_contiguous_equals_paged(name):
    from tests._replay import contiguous_layout
    wl = SMALL[name]()
    k, v, ctx = contiguous_layout(wl)
    got = A.contiguous_decode(wl.q, k, v, ctx, wl.scale, wl.dtype, wl.num_q_heads,
                              wl.num_kv_heads)
    assert np.array_equal(got, run_paged(wl))


def test_closed_forms():
    rng = np.random.default_rng(0)
    d = 16
    v = rng.standard_normal((9, d))
    k = rng.standard_normal((9, d))
    q = rng.standard_normal(d)
    # one token: the output is that token's V, exactly
    assert np.array_equal(A.decode_one(q, k[:1], v[:1], 0.25), v[0])
    # zero query (or all K equal): uniform weights, the mean of V
    assert np.allclose(A.decode_one(np.zeros(d), k, v, 0.25), v.mean(0), atol=1e-15)
    assert np.allclose(A.decode_one(q, np.tile(k[:1], (9, 1)), v, 0.25), v.mean(0), atol=1e-15)
    # constant V rows give that constant
    assert np.allclose(A.decode_one(q, k, np.full((9, d), 1.75), 0.25), 1.75, atol=1e-15)
    # a dominant score selects its V row
    kd = k.copy()
    kd[4] = 1e3 * q
    assert np.allclose(A.decode_one(q, kd, v, 1.0), v[4], atol=1e-12)
    # two equal top scores, the rest far below: the average of the two rows
    kd[7] = kd[4]
    assert np.allclose(A.decode_one(q, kd, v, 1.0), (v[4] + v[7]) / 2, atol=1e-12)


@pytest.mark.parametrize("name", ["gqa4_bf16_b4", "mha_shared_bf16", "beam_f16"])
def test_physical_relabelling_is_invisible(name):
    wl = SMALL[name]()
    other = np.random.default_rng(99).permutation(wl.num_blocks).astype(np.int32)
    a = run_paged(wl)
    b = run_paged(wl, free_order=other)
    t_a, _ = OracleRun(wl).tables(wl)
    t_b, _ = OracleRun(wl, other).tables(wl)
    assert not np.array_equal(t_a, t_b)
    assert np.array_equal(a, b)


def test_shared_prefix_equals_private_copies():
    mk = lambda share: W.shared_prefix("sp", 3, 4, 40, [1, 7, 9, 16, 30, 2, 5, 8, 11, 3, 4, 12],
                                       (8, 2, 16, 8, "bf16"), 128, 16, share=share, seed=8)
    shared, private = mk(True), mk(False)
    run_s, run_p = OracleRun(shared), OracleRun(private)
    assert run_s.pool.stats()["shared"] > 0 and run_p.pool.stats()["shared"] == 0
    assert np.array_equal(run_paged(shared), run_paged(private))


@pytest.mark.parametrize("partition", [1, 3, 8, 64, 100, 1000])
def test_split_combine_equals_one_pass(partition):
    rng = np.random.default_rng(partition)
    ctx, d = 777, 32
    q = rng.standard_normal(d)
    k = 3 * rng.standard_normal((ctx, d))
    v = rng.standard_normal((ctx, d))
    ref = A.decode_one(q, k, v, 0.2)
    assert np.max(np.abs(A.split_decode_one(q, k, v, 0.2, partition) - ref)) < 1e-13


# -- planted mistakes: each must be caught --------------------------------------

def _mutant(kind):
    def fn(q_bits, kc, vc, tables, lens, B, scale, dtype, Hq, Hkv):
        group = Hq // Hkv
        S, d = len(lens), q_bits.shape[-1]
        out = np.zeros((S, Hq, d))
        for s in range(S):
            ctx = int(lens[s]) - (kind == "ctx_minus_one")
            pos = np.arange(ctx)
            tab = np.asarray(tables[s], dtype=np.int64)
            blocks, rows = tab[pos // B], pos % B
            if kind == "row_block_swapped":
                blocks, rows = tab[np.minimum(pos % B, len(tab) - 1)], pos // B % B
            k = to_f64(kc[blocks, :, rows, :], dtype)
            v = to_f64(vc[blocks, :, rows, :], dtype)
            if kind == "k_v_swapped":
                k, v = v, k
            q = to_f64(q_bits[s], dtype)
            for h in range(Hq):
                g = h % Hkv if kind == "head_map_modulo" else h // group
                sc = 1.0 if kind == "no_scale" else scale
                z = sc * (k[:, g, :] @ q[h])
                if kind == "sign_flip":
                    z = -z
                w = np.exp(z - z.max())
                o = w @ v[:, g, :]
                out[s, h] = o if kind == "unnormalised" else o / w.sum()
        return out
    return fn


MUTANTS = ["ctx_minus_one", "row_block_swapped", "k_v_swapped", "head_map_modulo",
           "no_scale", "sign_flip", "unnormalised"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_attention_mistakes_are_caught(kind):
    caught = False
    for name in sorted(SMALL):
        wl = SMALL[name]()
        if kind == "head_map_modulo" and wl.num_q_heads == wl.num_kv_heads:
            continue
        got = run_paged(wl, fn=_mutant(kind))
        if not np.max(np.abs(got - sdpa_reference(wl))) < 1e-12:
            caught = True
            break
    assert caught, kind
    # the unmutated copy passes the same pin
    wl = SMALL["gqa4_bf16_b4"]()
    assert np.max(np.abs(run_paged(wl, fn=_mutant("none")) - sdpa_reference(wl))) < 1e-12
