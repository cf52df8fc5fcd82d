"""Comparison helpers shared by the CPU and GPU tests."""
import numpy as np


def rel_l2(x, ref):
    """||x - ref||_2 / ||ref||_2 over the whole tensor (fp64).  When the
    reference is exactly zero, returns max |x| instead."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.shape != ref.shape:
        raise ValueError(f"shape mismatch {x.shape} vs {ref.shape}")
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    if den == 0.0:
        return float(np.max(np.abs(x))) if x.size else 0.0
    return float(num / den)


# Parity gates, relative L2 on o and on the final state.
TOL_FP32 = 1e-4
TOL_BF16 = 2e-2
