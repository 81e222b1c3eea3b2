"""Decode raw floating-point bit patterns to float64 (test infrastructure).

The KV cache is held as raw bits on both sides of the parity check so that
cache contents can be compared bit for bit.  These decoders follow the IEEE
binary32 / binary16 definitions; bfloat16 is by definition the upper 16 bits
of a binary32, so widening it is a 16-bit left shift.
"""
import numpy as np

ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
BITS_DTYPE = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16}
# quiet-NaN patterns used to poison never-written cache slots
NAN_BITS = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0}


def to_f64(bits, dtype):
    """Raw bits (uint16 / uint32 array) -> float64 array of the same shape."""
    bits = np.asarray(bits)
    if dtype == "f32":
        return bits.astype(np.uint32).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        wide = bits.astype(np.uint32) << np.uint32(16)
        return wide.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")
