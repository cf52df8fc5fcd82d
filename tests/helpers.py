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


def _rel_from_sums(err2, ref2, absmax):
    """Relative L2 per group from summed squares; a group whose reference is
    exactly zero gets its max |x| (as rel_l2 does for a whole tensor)."""
    err2 = np.asarray(err2, dtype=np.float64)
    ref2 = np.asarray(ref2, dtype=np.float64)
    out = np.empty_like(err2)
    nz = ref2 > 0
    out[nz] = np.sqrt(err2[nz] / ref2[nz])
    out[~nz] = np.asarray(absmax, dtype=np.float64)[~nz]
    return out


def rel_l2_per_seq_head(o, ref, cu):
    """Relative L2 of each (sequence, head) block of a packed output.

    o, ref: [rows, H, dv]; cu: sequence offsets [N+1] into the rows.
    Returns an [N, H] array (NaN for empty sequences, which own no rows)."""
    o = np.asarray(o, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if o.shape != ref.shape or o.ndim != 3:
        raise ValueError(f"expected two [rows, H, dv] arrays, got {o.shape} and {ref.shape}")
    cu = np.asarray(cu, dtype=np.int64)
    N, H = len(cu) - 1, o.shape[1]
    err2_rows = np.sum((o - ref) ** 2, axis=-1)   # [rows, H]
    ref2_rows = np.sum(ref ** 2, axis=-1)
    abs_rows = np.max(np.abs(o), axis=-1)
    out = np.full((N, H), np.nan)
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        if b > a:
            out[n] = _rel_from_sums(err2_rows[a:b].sum(0), ref2_rows[a:b].sum(0), abs_rows[a:b].max(0))
    return out


def rel_l2_per_state(ht, ref):
    """Relative L2 of each [dk, dv] state of an [N, H, dk, dv] tensor; [N, H]."""
    ht = np.asarray(ht, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ht.shape != ref.shape or ht.ndim != 4:
        raise ValueError(f"expected two [N, H, dk, dv] arrays, got {ht.shape} and {ref.shape}")
    err2 = np.sum((ht - ref) ** 2, axis=(2, 3))
    ref2 = np.sum(ref ** 2, axis=(2, 3))
    return _rel_from_sums(err2, ref2, np.max(np.abs(ht), axis=(2, 3)))


def worst(per):
    """Largest entry of a per-(sequence, head) error table, ignoring NaN
    (empty sequences); 0 when there is none."""
    per = np.asarray(per, dtype=np.float64)
    return float(np.nanmax(per)) if np.any(np.isfinite(per)) else 0.0


# Parity gates, relative L2 on o and on the final state; the same gates
# apply to every (sequence, head) block on its own.
TOL_FP32 = 1e-4
TOL_BF16 = 2e-2
