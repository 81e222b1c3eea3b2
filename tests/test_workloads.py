"""The seeded generators are deterministic and match the stated recipes."""
import numpy as np

import workloads as W


def test_same_seed_same_bits():
    a, b = W.tiny(), W.tiny()
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k_rows, b.k_rows)
    assert np.array_equal(a.free_order, b.free_order)
    c = W.tiny(seed=1)
    assert not np.array_equal(a.q, c.q)


def test_sweep_draws_identical_qkv_for_every_block_size():
    ws = [W.block_sweep(B, batch=4, ctx=40) for B in (8, 16, 32)]
    for w in ws[1:]:
        assert np.array_equal(w.q, ws[0].q)
        assert np.array_equal(w.k_rows, ws[0].k_rows)
        assert np.array_equal(w.v_rows, ws[0].v_rows)


def test_recipe_shapes():
    t = W.tiny()
    assert t.info["ctx"] == [7, 19, 33, 64] and t.num_blocks == 32 and t.dtype == "f32"
    assert sorted(t.free_order.tolist()) == list(range(32))
    x = W.gqa_suffix_lengths(0, 256)
    assert x.min() >= 1 and x.max() <= 8192 - 1008
    # lognormal with mean 512: the sample mean of 256 draws sits near it
    assert 350 < x.mean() < 700
    rs = W.synth._streams(0)
    ctx = rs["lengths"].integers(128, 2048, size=64, endpoint=True)
    assert ctx.min() >= 128 and ctx.max() <= 2048


def test_bf16_rounding_is_nearest_even():
    # 1 + 2^-8 is halfway between bf16 neighbours 1 and 1 + 2^-7: ties to even (1.0)
    import torch
    x = torch.tensor([1 + 2 ** -8, 1 + 3 * 2 ** -8], dtype=torch.float32)
    bits = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert bits.tolist() == [0x3F80, 0x3F82]
