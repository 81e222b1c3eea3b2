"""Output tolerances for the decode parity tests.

16-bit inputs with float32 accumulation: max-abs error <= 2e-3 and relative
L2 error <= 1e-3 against the float64 oracle.  float32 inputs: 1e-5 for both
(the kernel's float32 dot products and sums over <= 8192 tokens stay far
inside it).
"""
import numpy as np

TOL = {"f32": (1e-5, 1e-5), "f16": (2e-3, 1e-3), "bf16": (2e-3, 1e-3)}


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    max_abs = float(np.max(np.abs(got - ref))) if got.size else 0.0
    rel_l2 = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    return max_abs, rel_l2


def assert_close(got, ref, dtype, what=""):
    max_abs, rel_l2 = errors(got, ref)
    ta, tr = TOL[dtype]
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert max_abs <= ta and rel_l2 <= tr, f"{what}: max_abs {max_abs:.3g} rel_l2 {rel_l2:.3g}"
    return max_abs, rel_l2
