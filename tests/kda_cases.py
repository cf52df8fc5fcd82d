"""Shared helpers for the parity tests: run the HIP path and the oracle on the
same seeded inputs and compare with relative L2, over the whole tensors and
over every (sequence, head) block on its own."""
import numpy as np
import torch

import oracle
import workloads
from helpers import TOL_BF16, TOL_FP32, rel_l2, rel_l2_per_seq_head, rel_l2_per_state, worst


def tol_for(dtype_name):
    return TOL_FP32 if dtype_name == "fp32" else TOL_BF16


def seq_offsets(x):
    """Sequence offsets [N+1] into the packed rows of a prefill batch."""
    B, T = x["q"].shape[:2]
    return (x["cu_seqlens"].cpu().numpy().astype(np.int64) if x["cu_seqlens"] is not None
            else np.arange(B + 1, dtype=np.int64) * T)


def packed_view(x):
    """(q, k, v, g, beta, cu) as packed [rows, H, d] float32 numpy arrays."""
    B, T = x["q"].shape[:2]
    f = lambda t: workloads.to_numpy_f32(t).reshape((B * T,) + tuple(t.shape[2:]))
    return f(x["q"]), f(x["k"]), f(x["v"]), f(x["g"]), f(x["beta"]), seq_offsets(x)


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


def gate(o, o_ref, ht, ht_ref, cu, tol, what="", block_tol=None):
    """Whole-tensor and per-(sequence, head) rel-L2 of o [rows, H, dv] and ht
    [N, H, dk, dv] against the oracle; asserts the whole-tensor figures <=
    tol and every block's <= block_tol (tol unless a case states a looser
    one), and returns (o, ht, worst o block, worst ht block)."""
    block_tol = tol if block_tol is None else block_tol
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ht)), f"{what}: non-finite output"
    eo, eh = rel_l2(o, o_ref), rel_l2(ht, ht_ref)
    wo = worst(rel_l2_per_seq_head(o, o_ref, cu))
    wh = worst(rel_l2_per_state(ht, ht_ref))
    print(f"[parity]   {what} rel-L2 o={eo:.3e} ht={eh:.3e}; worst (sequence, head) o={wo:.3e} "
          f"ht={wh:.3e} (tol {tol:g}, per block {block_tol:g})", flush=True)
    assert eo <= tol, f"o rel-L2 {eo:.3e} > {tol}"
    assert eh <= tol, f"ht rel-L2 {eh:.3e} > {tol}"
    assert wo <= block_tol, f"worst (sequence, head) o rel-L2 {wo:.3e} > {block_tol}"
    assert wh <= block_tol, f"worst (sequence, head) ht rel-L2 {wh:.3e} > {block_tol}"
    return eo, eh, wo, wh


def check_prefill(spec, chunk=None, label="", block_tol=None, **kw):
    """GPU vs oracle on the whole output and final state and on every
    (sequence, head) block; returns the four errors."""
    x = workloads.make_prefill(spec)
    chunk = chunk or spec.chunk
    print(f"[parity] {label or spec} chunk={chunk}", flush=True)
    o, ht = gpu_prefill(x, chunk, **kw)
    o_ref, ht_ref = oracle_prefill(x)
    B, T = x["q"].shape[:2]
    o_ref = o_ref.reshape((B * T,) + o_ref.shape[-2:])
    return gate(to_np64(o).reshape(o_ref.shape), o_ref, to_np64(ht), ht_ref, seq_offsets(x), tol_for(spec.dtype),
                label, block_tol)
