"""8-bit float (E4M3) KV-cache codes and decode over them (test infrastructure).

Test infrastructure only; the parity tests compare the codes pa_write_kv_fp8
writes and the output of FP8 decode against this module.

Why: PagedAttention removes fragmentation but not the byte floor of the KV
cache; fewer bytes come from GQA, a quantised KV cache or shorter contexts
("Paged Attention" (daiw.org), 量化, the warning box), and serving systems
ship FP8 quantisation ("vLLM PagedAttention：大模型推理的显存管理革命"
(horeb.top), 生态现状).  The pages fix no format; the readings taken here:

* E4M3 as in the OCP 8-bit floating point specification, "FN" variant: 1 sign
  bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 holds the
  subnormals m/8 * 2^-6; code 0x7F / 0xFF is NaN and there are no
  infinities, so the largest finite value is 1.75 * 2^8 = 448.
* One float32 scale per cache (K and V each): the stored code is the E4M3
  value nearest to x * (1 / scale), computed in float32 (the reciprocal
  rounded to float32 once, the product rounded to float32), ties to the even
  code; magnitudes at or beyond 448 saturate to +-448 and NaN stays NaN.
* Decoding a code gives value(code) * scale exactly (float64 here).

quantize() works from the definition: it finds the nearest entry of the
value table, with no bit manipulation that could hide an off-by-one.
"""
import numpy as np

from .attention import decode_one
from .bits import to_f64


def e4m3_value(code):
    """Value of one E4M3 code (float64; NaN for 0x7F / 0xFF)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


VALUES = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
MAX_FINITE = 448.0
_POS = VALUES[:0x7F]          # codes 0x00 .. 0x7E: 0, increasing up to 448


def _nearest_code(a):
    """Codes (0..0x7E) of the values nearest to magnitudes a (finite, < 448),
    ties to the even code."""
    hi = np.searchsorted(_POS, a, side="left")          # first value >= a
    hi = np.minimum(hi, len(_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    return np.where(pick_hi, hi, lo).astype(np.uint8)


def encode(y):
    """float32 values -> E4M3 codes (nearest, ties to even, saturating)."""
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    out = np.empty(y.shape, dtype=np.uint8)
    nan = np.isnan(y)
    a = np.where(nan, 0.0, np.abs(y))
    sat = a >= MAX_FINITE
    mag = np.where(sat, 0x7E, _nearest_code(np.where(sat, 0.0, a)))
    sign = np.where(np.signbit(y), 0x80, 0)
    out[...] = (mag | sign).astype(np.uint8)
    out[nan] = 0x7F
    return out


def inv_scale(scale):
    """The float32 reciprocal both sides multiply by."""
    return np.float32(1.0) / np.float32(scale)


def quantize(x, scale):
    """Codes of x (float32-exact values) under scale: encode(f32(x * f32(1/scale)))."""
    y = np.asarray(x, dtype=np.float32) * inv_scale(scale)       # one float32 rounding
    return encode(y.astype(np.float32))


def quantize_bits16(bits, dtype, scale):
    """quantize() of 16-bit inputs given as raw bits ("f16" or "bf16"): the
    codes of all 65536 patterns are computed once with quantize() itself,
    then looked up, which is the same function over any array of them."""
    from .bits import to_f64
    table = quantize(to_f64(np.arange(65536, dtype=np.uint16), dtype).astype(np.float32), scale)
    return table[np.asarray(bits, dtype=np.uint16)]


def dequantize(codes, scale):
    return VALUES[np.asarray(codes, dtype=np.uint8)] * float(np.float32(scale))


def paged_decode_fp8(q_bits, q_dtype, k_codes, v_codes, k_scale, v_scale, block_tables, ctx_lens,
                     block_size, scale, num_q_heads, num_kv_heads, heads=None):
    """Decode attention through block tables over an E4M3 cache.

    q_bits        ``[S][Hq][d]`` raw bits of q_dtype
    k/v_codes     ``[num_blocks][Hkv][B][d]`` uint8 codes
    Returns float64 ``[S][Hq][d]``: each row is softmax(scale q.K) V with K, V
    the dequantised codes (value(code) * scale of the cache).
    """
    S = len(ctx_lens)
    d = q_bits.shape[-1]
    group = num_q_heads // num_kv_heads
    out = np.zeros((S, num_q_heads, d), dtype=np.float64)
    want = None
    if heads is not None:
        want = {}
        for s, h in heads:
            want.setdefault(int(s), []).append(int(h))
    for s in range(S):
        if want is not None and s not in want:
            continue
        ctx = int(ctx_lens[s])
        if ctx <= 0:
            continue
        pos = np.arange(ctx)
        blocks = np.asarray(block_tables[s], dtype=np.int64)[pos // block_size]
        rows = pos % block_size
        k = dequantize(k_codes[blocks, :, rows, :], k_scale)     # [ctx][Hkv][d]
        v = dequantize(v_codes[blocks, :, rows, :], v_scale)
        q = to_f64(q_bits[s], q_dtype)
        for h in (want[s] if want is not None else range(num_q_heads)):
            g = h // group
            out[s, h] = decode_one(q[h], k[:, g, :], v[:, g, :], scale)
    return out
