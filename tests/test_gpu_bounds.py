"""No store past the end of o or ht (needs a GPU).  o and ht are the leading
part of larger buffers filled with a sentinel; after the call every
sentinel byte past them must be unchanged, and the outputs must still match
the oracle.  Ragged last chunks pad their rows past the sequence end with
neutral tokens; each kernel path (the loader-fed state chain, the
register-fed chain, the segment output chains of both dtypes, packed
sequences) must drop those rows instead of storing them."""
import pytest
import torch

import workloads
from kda_cases import gate, oracle_prefill, seq_offsets, to_np64, tol_for

pytestmark = pytest.mark.gpu

Spec = workloads.PrefillSpec
PAD = 1 << 16  # sentinel elements past each output

CASES = [
    ("loader-fed chain", Spec(H=2, dk=128, dv=128, T=100, B=2, dtype="bf16", chunk=64, h0_std=1.0,
                              g_mode="slow", seed=91), 0),
    ("register-fed chain", Spec(H=3, dk=64, dv=128, T=77, B=2, dtype="bf16", chunk=64, h0_std=1.0,
                                g_mode="slow", seed=92), 0),
    ("segmented bf16", Spec(H=1, dk=128, dv=128, T=64 * 64 + 5, B=1, dtype="bf16", chunk=64, h0_std=1.0,
                            g_mode="slow", seed=93), 0),
    ("segmented bf16 dv64", Spec(H=1, dk=128, dv=64, T=64 * 64 + 9, B=1, dtype="bf16", chunk=64, h0_std=1.0,
                                 g_mode="slow", seed=94), 0),
    ("segmented fp32", Spec(H=1, dk=32, dv=32, T=2048 + 3, B=1, dtype="fp32", chunk=16, h0_std=1.0,
                            g_mode="slow", seed=95), 0),
    ("packed", Spec(H=2, dk=128, dv=128, seqlens=(70, 1, 0, 129, 33), dtype="bf16", chunk=64, h0_std=1.0,
                    g_mode="slow", seed=96), 0),
    ("single chain, flag", Spec(H=1, dk=128, dv=128, T=64 * 64 + 5, B=1, dtype="bf16", chunk=64, h0_std=1.0,
                                g_mode="slow", seed=97), 2),
]


def _sentinel_like(shape, dtype, dev):
    """A flat buffer of prod(shape) + PAD elements of a fixed bit pattern, and
    the leading view of ``shape``."""
    n = 1
    for s in shape:
        n *= s
    bits = torch.int16 if dtype == torch.bfloat16 else torch.int32
    raw = torch.full((n + PAD,), 0x3a5c if bits == torch.int16 else 0x3a5c7e11, dtype=bits, device=dev)
    buf = raw.view(dtype)
    return raw, buf[:n].view(shape), n


@pytest.mark.parametrize("label,spec,flags", CASES, ids=[c[0] for c in CASES])
def test_no_store_past_outputs(label, spec, flags):
    import gated_delta_rule_97_amd as kda
    x = workloads.make_prefill(spec)
    d = {key: (val.cuda() if val is not None else None) for key, val in x.items()}
    B, T, H = d["q"].shape[0], d["q"].shape[1], spec.H
    dt = d["q"].dtype
    raw_o, o, no = _sentinel_like((B, T, H, spec.dv), dt, "cuda")
    raw_h, ht, nh = _sentinel_like((spec.num_seqs, H, spec.dk, spec.dv), torch.float32, "cuda")
    tail_o, tail_h = raw_o[no:].clone(), raw_h[nh:].clone()
    print(f"[bounds] {label}", flush=True)
    kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"], chunk_size=spec.chunk,
                      o=o, ht=ht, flags=flags)
    torch.cuda.synchronize()
    assert torch.equal(raw_o[no:], tail_o), f"{label}: a store landed past the end of o"
    assert torch.equal(raw_h[nh:], tail_h), f"{label}: a store landed past the end of ht"
    o_ref, ht_ref = oracle_prefill(x)
    gate(to_np64(o).reshape(o_ref.shape), o_ref, to_np64(ht), ht_ref, seq_offsets(x), tol_for(spec.dtype), label)
