"""Pins of the E4M3 oracle (CPU only).

The value table is checked against facts of the format definition (largest
finite 448, smallest normal 2^-6, smallest subnormal 2^-9, 1.0, NaN codes,
signed zero); quantisation is checked bit for bit against torch's float8
e4m3fn conversion on in-range values (random, exact midpoints between
neighbours, subnormals), against round trips of every code, saturation,
monotonicity and the half-step error bound; decode over codes is checked
against the float32 decode oracle on caches holding the same values.
Planted mistakes (ties away from zero, no saturation, the scale not applied
in quantisation) must fail.
"""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import fp8 as F


def test_value_table_matches_the_definition():
    V = F.VALUES
    assert V[0x7E] == 448.0 and V[0xFE] == -448.0
    assert V[0x08] == 2.0 ** -6 and V[0x07] == 7 / 8 * 2.0 ** -6
    assert V[0x01] == 2.0 ** -9
    assert V[0x38] == 1.0 and V[0x40] == 2.0 and V[0x39] == 1.125
    assert np.isnan(V[0x7F]) and np.isnan(V[0xFF])
    assert V[0x00] == 0.0 and V[0x80] == 0.0 and np.signbit(V[0x80])
    pos = V[:0x7F]
    assert np.all(np.diff(pos) > 0)                    # codes 0..0x7E increase
    assert np.sum(np.isfinite(V)) == 254


def torch_codes(y):
    return torch.from_numpy(np.asarray(y, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_matches_torch_in_range():
    rng = np.random.default_rng(0)
    y = np.concatenate([
        rng.normal(0, 30, 20000), rng.uniform(-448, 448, 20000),
        rng.normal(0, 2.0 ** -7, 5000),                              # subnormal range
        (F.VALUES[1:0x7E] + F.VALUES[2:0x7F]) / 2,                   # exact midpoints: ties
        -(F.VALUES[1:0x7E] + F.VALUES[2:0x7F]) / 2,
        F.VALUES[:0x7F], -F.VALUES[1:0x7F],
    ]).astype(np.float32)
    y = y[np.abs(y) <= 448]
    assert np.array_equal(F.encode(y), torch_codes(y))


def test_every_code_round_trips_and_out_of_range_saturates():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(F.encode(F.VALUES[codes].astype(np.float32)), codes)
    big = np.array([448.0, 449.0, 463.9, 464.0, 480.0, 1e6, np.float32(3.4e38)], dtype=np.float32)
    assert np.all(F.encode(big) == 0x7E) and np.all(F.encode(-big) == 0xFE)
    assert F.encode(np.array([np.nan], dtype=np.float32))[0] == 0x7F


def test_monotone_and_within_half_a_step():
    y = np.sort(np.random.default_rng(1).uniform(-440, 440, 50000).astype(np.float32))
    v = F.VALUES[F.encode(y)]
    assert np.all(np.diff(v) >= 0)
    a = np.abs(y.astype(np.float64))
    step = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))
    assert np.all(np.abs(v - y) <= step / 2)


def test_quantize_uses_the_float32_reciprocal():
    x = np.array([1.0, 3.0, 100.0, -7.5], dtype=np.float32)
    s = 0.3
    inv = np.float32(1) / np.float32(s)
    assert np.array_equal(F.quantize(x, s), F.encode((x * inv).astype(np.float32)))
    assert np.allclose(F.dequantize(F.quantize(x, s), s), x, rtol=2 ** -4)


def test_decode_over_codes_equals_the_float32_oracle():
    rng = np.random.default_rng(2)
    nb, hkv, B, d, S, G = 12, 2, 8, 16, 3, 2
    kc = rng.integers(0, 256, size=(nb, hkv, B, d)).astype(np.uint8)
    vc = rng.integers(0, 256, size=(nb, hkv, B, d)).astype(np.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x38                 # no NaN codes
    vc[(vc & 0x7F) == 0x7F] = 0x38
    tables = np.array([rng.permutation(nb)[:4] for _ in range(S)])
    ctx = np.array([5, 31, 17])
    q = rng.normal(0, 0.05, size=(S, G * hkv, d)).astype(np.float32)
    got = F.paged_decode_fp8(q.view(np.uint32), "f32", kc, vc, 1.0, 1.0, tables, ctx, B, 0.25, G * hkv, hkv)
    kf = F.VALUES[kc].astype(np.float32).view(np.uint32)
    vf = F.VALUES[vc].astype(np.float32).view(np.uint32)
    ref = A.paged_decode(q.view(np.uint32), kf, vf, tables, ctx, B, 0.25, "f32", G * hkv, hkv)
    assert np.array_equal(got, ref)
    # the scales multiply the cached values
    got2 = F.paged_decode_fp8(q.view(np.uint32), "f32", kc, vc, 1.0, 2.0, tables, ctx, B, 0.25, G * hkv, hkv)
    assert np.allclose(got2, 2 * ref, rtol=1e-12)


@pytest.mark.parametrize("mutant", ["ties_away", "no_saturation", "scale_ignored"])
def test_planted_mistakes_fail(mutant, monkeypatch):
    if mutant == "ties_away":
        def nearest(a):
            hi = np.minimum(np.searchsorted(F._POS, a, side="left"), len(F._POS) - 1)
            lo = np.maximum(hi - 1, 0)
            return np.where(F._POS[hi] - a <= a - F._POS[lo], hi, lo).astype(np.uint8)
        monkeypatch.setattr(F, "_nearest_code", nearest)
        with pytest.raises(AssertionError):
            test_encode_matches_torch_in_range()
    elif mutant == "no_saturation":
        orig = F.encode

        def enc(y):
            out = orig(y)
            out[np.abs(np.asarray(y, dtype=np.float32)) >= 448] = 0x7F
            return out
        monkeypatch.setattr(F, "encode", enc)
        with pytest.raises(AssertionError):
            test_every_code_round_trips_and_out_of_range_saturates()
    else:
        monkeypatch.setattr(F, "inv_scale", lambda s: np.float32(1.0))
        with pytest.raises(AssertionError):
            test_quantize_uses_the_float32_reciprocal()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_quantize_bits16_equals_quantize(dtype):
    # the table path must be quantize() itself: every pattern, and a random array
    from oracle.bits import to_f64
    every = np.arange(65536, dtype=np.uint16)
    for scale in (1 / 56, 0.5, 3.0):
        assert np.array_equal(F.quantize_bits16(every, dtype, scale),
                              F.quantize(to_f64(every, dtype).astype(np.float32), scale))
    bits = np.random.default_rng(3).integers(0, 65536, size=(7, 3, 16, 8), dtype=np.uint16)
    assert np.array_equal(F.quantize_bits16(bits, dtype, 1 / 72),
                          F.quantize(to_f64(bits, dtype).astype(np.float32), 1 / 72))
