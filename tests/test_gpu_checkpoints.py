"""Strided state checkpoints of the prefill (needs a GPU), against the fp64
oracle: checkpoint j of a sequence is the oracle's final state after that
sequence's first (j + 1) * stride tokens, from the same initial state.  The
outputs o and ht of the checkpointed call are bit-identical to the plain
call's (the checkpoints are extra stores of the same state)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import TOL_BF16, rel_l2
from kda_cases import packed_view, to_np64, tol_for

pytestmark = pytest.mark.gpu

Spec = workloads.PrefillSpec


def ref_checkpoints(x, stride, only=None):
    """Oracle states after every full stride of every sequence, in the
    library's slot order; ``only`` = slot indices to compute (others NaN)."""
    q, k, v, g, b, cu = packed_view(x)
    h0 = None if x["h0"] is None else x["h0"].cpu().numpy().astype(np.float64)
    H, dk, dv = q.shape[1], q.shape[2], v.shape[2]
    slots = []  # (sequence, prefix length)
    for n in range(len(cu) - 1):
        for j in range((cu[n + 1] - cu[n]) // stride):
            slots.append((n, (j + 1) * stride))
    want = range(len(slots)) if only is None else only
    rows, lens, seqs = [], [], []
    for i in want:
        n, L = slots[i]
        rows.append(np.arange(cu[n], cu[n] + L))
        lens.append(L)
        seqs.append(n)
    out = np.full((len(slots), H, dk, dv), np.nan)
    if not seqs:
        return out
    r = np.concatenate(rows)
    cu2 = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    h02 = None if h0 is None else h0[seqs]
    _, ht = oracle.prefill(q[r], k[r], v[r], g[r], b[r], h02, cu2)
    out[list(want)] = ht
    return out


def run(x, chunk, stride, **kw):
    import gated_delta_rule_97_amd as kda
    d = {key: (val.cuda() if val is not None else None) for key, val in x.items()}
    res = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"],
                            chunk_size=chunk, ckpt_stride=stride, **kw)
    plain = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"],
                              chunk_size=chunk)
    torch.cuda.synchronize()
    return res, plain


CASES = [
    ("fixed bf16", Spec(H=3, dk=128, dv=128, T=700, B=2, dtype="bf16", chunk=64, h0_std=1.0, g_mode="slow",
                        seed=51), 64, 128),
    ("fixed bf16 d=64/32", Spec(H=2, dk=64, dv=32, T=512, B=3, dtype="bf16", chunk=64, h0_std=1.0,
                                g_mode="slow", seed=52), 64, 64),
    ("packed bf16", Spec(H=2, dk=128, dv=64, seqlens=(37, 0, 512, 129, 300, 64), dtype="bf16", chunk=64,
                         h0_std=1.0, g_mode="slow", seed=53), 64, 64),
    ("packed fp32 chunk 16", Spec(H=2, dk=32, dv=64, seqlens=(5, 48, 0, 33, 96), dtype="fp32", chunk=16,
                                  h0_std=1.0, g_mode="slow", seed=54), 16, 32),
]


@pytest.mark.parametrize("label,spec,chunk,stride", CASES, ids=[c[0] for c in CASES])
def test_checkpoints_match_oracle_prefix_states(label, spec, chunk, stride):
    x = workloads.make_prefill(spec)
    print(f"[parity] checkpoints {label} stride={stride}", flush=True)
    (o, ht, ck), (o2, ht2) = run(x, chunk, stride)
    assert torch.equal(o, o2) and torch.equal(ht, ht2)
    ref = ref_checkpoints(x, stride)
    assert ck.shape[0] == ref.shape[0]
    if ref.shape[0]:
        e = rel_l2(to_np64(ck), ref)
        print(f"[parity]   {ref.shape[0]} checkpoints, rel-L2 {e:.3e}", flush=True)
        assert e <= tol_for(spec.dtype)
        # per-checkpoint too: a misplaced slot would hide in the global norm
        for i in range(ref.shape[0]):
            assert rel_l2(to_np64(ck[i]), ref[i]) <= tol_for(spec.dtype), f"slot {i}"


def test_fewer_slots_are_not_overrun():
    """A ckpt buffer with fewer slots than checkpoints gets only those; the
    memory after it is untouched."""
    spec = Spec(H=2, dk=64, dv=64, T=512, B=2, dtype="bf16", chunk=64, h0_std=1.0, g_mode="slow", seed=55)
    x = workloads.make_prefill(spec)
    buf = torch.full((6, 2, 64, 64), 7.0, device="cuda")  # 8 checkpoints exist; give 5 slots + a guard
    (o, ht, ck), _ = run(x, 64, 128, ckpt=buf[:5])
    assert torch.all(buf[5] == 7.0)
    ref = ref_checkpoints(x, 128, only=range(5))
    assert rel_l2(to_np64(buf[:5]), ref[:5]) <= TOL_BF16


def test_resume_from_checkpoint():
    """Prefix-cache use: prefill(rest, h0 = checkpoint) continues the
    sequence exactly as the uninterrupted call."""
    import gated_delta_rule_97_amd as kda
    spec = Spec(H=4, dk=128, dv=128, T=1024, B=1, dtype="bf16", chunk=64, h0_std=1.0, g_mode="slow", seed=56)
    x = workloads.make_prefill(spec)
    (o, ht, ck), _ = run(x, 64, 256)
    d = {key: (val.cuda() if val is not None else None) for key, val in x.items()}
    cut = 512  # checkpoint 1
    rest = lambda t: t[:, cut:].contiguous()
    o_r, ht_r = kda.chunk_prefill(rest(d["q"]), rest(d["k"]), rest(d["v"]), rest(d["g"]), rest(d["beta"]),
                                  ck[1:2].contiguous())
    torch.cuda.synchronize()
    assert rel_l2(to_np64(o_r), to_np64(o[:, cut:])) <= TOL_BF16
    assert rel_l2(to_np64(ht_r), to_np64(ht)) <= TOL_BF16


def test_headline_checkpoints_sampled():
    """The headline prefill (H=32, T=8192, d=128, bf16, chunk 64) with a
    checkpoint every 512 tokens: 16 per head; the oracle checks three."""
    spec = workloads.PREFILL_H32_T8K
    x = workloads.make_prefill(spec)
    (o, ht, ck), (o2, ht2) = run(x, 64, 512)
    assert torch.equal(o, o2) and torch.equal(ht, ht2)
    assert ck.shape[0] == 16
    only = [0, 7, 15]
    ref = ref_checkpoints(x, 512, only=only)
    for i in only:
        e = rel_l2(to_np64(ck[i]), ref[i])
        print(f"[parity]   headline checkpoint {i}: rel-L2 {e:.3e}", flush=True)
        assert e <= TOL_BF16
    assert torch.equal(ck[15], ht[0])  # 8192 = 16 x 512: the last checkpoint is the final state


@pytest.mark.parametrize("chunk,stride,T", [(16, 16, 100), (64, 64, 200), (64, 192, 700)])
def test_checkpoint_every_chunk_and_uneven_strides(chunk, stride, T):
    """A checkpoint after every chunk, and a stride of three chunks that does
    not divide the length (the trailing partial stride has no checkpoint)."""
    spec = Spec(H=2, dk=64, dv=64, T=T, B=2, dtype="bf16", chunk=chunk, h0_std=1.0, g_mode="slow", seed=57)
    x = workloads.make_prefill(spec)
    (o, ht, ck), (o2, ht2) = run(x, chunk, stride)
    assert torch.equal(o, o2) and torch.equal(ht, ht2)
    ref = ref_checkpoints(x, stride)
    assert ck.shape[0] == ref.shape[0] == 2 * (T // stride)
    for i in range(ref.shape[0]):
        assert rel_l2(to_np64(ck[i]), ref[i]) <= TOL_BF16, f"slot {i}"
