"""Shared helpers for the parity tests: run the HIP path and the oracle on the
same seeded inputs and compare with relative L2."""
import numpy as np
import torch

import oracle
import workloads
from helpers import TOL_BF16, TOL_FP32, rel_l2


def tol_for(dtype_name):
    return TOL_FP32 if dtype_name == "fp32" else TOL_BF16


def packed_view(x):
    """(q, k, v, g, beta, cu) as packed [rows, H, d] float32 numpy arrays."""
    B, T = x["q"].shape[:2]
    f = lambda t: workloads.to_numpy_f32(t).reshape((B * T,) + tuple(t.shape[2:]))
    cu = (x["cu_seqlens"].cpu().numpy().astype(np.int64) if x["cu_seqlens"] is not None
          else np.arange(B + 1, dtype=np.int64) * T)
    return f(x["q"]), f(x["k"]), f(x["v"]), f(x["g"]), f(x["beta"]), cu


def oracle_prefill(x, seqs=None):
    """fp64 oracle on the packed view; ``seqs`` restricts to some sequences
    (returns o rows of those sequences only, concatenated, and their ht)."""
    q, k, v, g, b, cu = packed_view(x)
    h0 = None if x["h0"] is None else x["h0"].cpu().numpy().astype(np.float64)
    if seqs is None:
        return oracle.prefill(q, k, v, g, b, h0, cu)
    rows = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in seqs]).astype(np.int64)
    lens = [cu[n + 1] - cu[n] for n in seqs]
    cu2 = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    h02 = None if h0 is None else h0[list(seqs)]
    return oracle.prefill(q[rows], k[rows], v[rows], g[rows], b[rows], h02, cu2)


def gpu_prefill(x, chunk, **kw):
    import gated_delta_rule_97_amd as kda
    d = {key: (val.cuda() if val is not None else None) for key, val in x.items()}
    o, ht = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"],
                              chunk_size=chunk, **kw)
    torch.cuda.synchronize()
    return o, ht


def to_np64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def check_prefill(spec, chunk=None, label=""):
    """GPU vs oracle on the whole output and final state; returns the errors."""
    x = workloads.make_prefill(spec)
    chunk = chunk or spec.chunk
    print(f"[parity] {label or spec} chunk={chunk}", flush=True)
    o, ht = gpu_prefill(x, chunk)
    o_ref, ht_ref = oracle_prefill(x)
    B, T = x["q"].shape[:2]
    eo = rel_l2(to_np64(o).reshape(o_ref.shape), o_ref)
    eh = rel_l2(to_np64(ht), ht_ref)
    tol = tol_for(spec.dtype)
    print(f"[parity]   rel-L2 o={eo:.3e} ht={eh:.3e} (tol {tol:g})", flush=True)
    assert np.all(np.isfinite(to_np64(o))) and np.all(np.isfinite(to_np64(ht)))
    assert eo <= tol, f"o rel-L2 {eo:.3e} > {tol}"
    assert eh <= tol, f"ht rel-L2 {eh:.3e} > {tol}"
    return eo, eh
