"""kda_chunk_prefill_noalloc through the C ABI (needs a GPU).

Three calls in a row on the one static scratch array, each smaller than the
one before: 16 heads x 4096 tokens (the loader-fed chain), then one long
sequence of 2 heads (the segment-parallel chain, its scratch written over
the first call's), then a packed batch.  Each must give exactly what
kda_chunk_prefill gives with a workspace of its own (the same kernels, so
bit-identical), and match the fp64 oracle at the parity gates.  A size past
the static limit is refused with nothing launched."""
import pytest
import torch

import workloads
from kda_cases import gate, oracle_prefill, seq_offsets, to_np64, tol_for

pytestmark = pytest.mark.gpu

Spec = workloads.PrefillSpec

CALLS = [
    ("16 heads x 4096 tokens", Spec(H=16, dk=128, dv=128, T=4096, B=1, dtype="bf16", chunk=64, h0_std=1.0,
                                    g_mode="slow", seed=121)),
    ("segmented 2 heads x 4133 tokens", Spec(H=2, dk=128, dv=128, T=64 * 64 + 37, B=1, dtype="bf16", chunk=64,
                                             h0_std=1.0, g_mode="slow", seed=122)),
    ("packed", Spec(H=3, dk=64, dv=128, seqlens=(70, 0, 1, 129, 33), dtype="bf16", chunk=64, h0_std=1.0,
                    g_mode="slow", seed=123)),
]


def _ptr(t):
    return 0 if t is None else t.data_ptr()


def _noalloc(kda, d, spec, o, ht):
    B, T, H = d["q"].shape[0], d["q"].shape[1], spec.H
    return kda.kda_chunk_prefill_noalloc(
        _ptr(d["q"]), _ptr(d["k"]), _ptr(d["v"]), _ptr(d["g"]), _ptr(d["beta"]), _ptr(d["h0"]),
        _ptr(d["cu_seqlens"]), B, T, H, spec.dk, spec.dv, spec.num_seqs, spec.chunk, kda.KDA_DTYPE_BF16, 0,
        _ptr(o), _ptr(ht), torch.cuda.current_stream().cuda_stream)


def test_noalloc_matches_the_workspace_entry_point():
    import gated_delta_rule_97_amd as kda
    for label, spec in CALLS:
        x = workloads.make_prefill(spec)
        d = {key: (val.cuda() if val is not None else None) for key, val in x.items()}
        B, T = d["q"].shape[:2]
        need = kda.workspace_bytes(B, T, spec.H, spec.dk, spec.dv, spec.num_seqs, spec.chunk, kda.KDA_DTYPE_BF16)
        assert need <= kda.NOALLOC_SCRATCH_BYTES, label
        print(f"[noalloc] {label}: workspace {need} B", flush=True)
        o_ws, ht_ws = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"],
                                        chunk_size=spec.chunk)
        o = torch.full_like(o_ws, float("nan"))
        ht = torch.full_like(ht_ws, float("nan"))
        st = _noalloc(kda, d, spec, o, ht)
        assert st == kda.KDA_OK, kda.kda_status_string(st)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ws), f"{label}: o differs from kda_chunk_prefill's"
        assert torch.equal(ht, ht_ws), f"{label}: ht differs from kda_chunk_prefill's"
        o_ref, ht_ref = oracle_prefill(x)
        gate(to_np64(o).reshape(o_ref.shape), o_ref, to_np64(ht), ht_ref, seq_offsets(x), tol_for(spec.dtype),
             label)


def test_noalloc_refuses_sizes_past_its_scratch():
    import gated_delta_rule_97_amd as kda
    spec = Spec(H=32, dk=128, dv=128, T=4096, B=1, dtype="bf16", chunk=64, seed=124)
    d = {key: (val.cuda() if val is not None else None) for key, val in workloads.make_prefill(spec).items()}
    o = torch.full((1, 4096, 32, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    ht = torch.full((1, 32, 128, 128), -1.0, dtype=torch.float32, device="cuda")
    assert _noalloc(kda, d, spec, o, ht) == kda.KDA_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert bool((o == 3.0).all()) and bool((ht == -1.0).all()), "a refused call launches nothing"
