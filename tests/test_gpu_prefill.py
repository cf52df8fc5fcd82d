"""Parity of the HIP chunked prefill against the fp64 oracle (needs a GPU).

Inputs follow the workload recipe (workloads/); the oracle consumes the exact
bf16 / fp32 values the GPU sees.  Gates: relative L2 <= 1e-4 (fp32 inputs),
<= 2e-2 (bf16 inputs with fp32 accumulation), on o and on the final state,
over the whole tensors and over every (sequence, head) block on its own.
Stress variants (slow decay, state isolation, g at the -5 floor, no decay)
run because at the configs' own decay the state remembers only a few
tokens, so a broken inter-chunk carry would otherwise pass.
"""
import numpy as np
import pytest
import torch

import workloads
from helpers import TOL_BF16, TOL_FP32, rel_l2
from kda_cases import check_prefill, gpu_prefill, oracle_prefill, to_np64

pytestmark = pytest.mark.gpu

Spec = workloads.PrefillSpec


def test_tiny_fp32_config():
    """The tiny fp32 workload: B=1, H=2, T=64, d=32, chunk 16."""
    check_prefill(workloads.TINY_FP32, label="tiny fp32")


@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("chunk", [16, 64])
def test_bf16_shapes_ragged(dk, dv, chunk):
    """Several tiles and a ragged tail (T = 200 is not a multiple of 16 or 64)."""
    spec = Spec(H=3, dk=dk, dv=dv, T=200, B=2, dtype="bf16", chunk=chunk, h0_std=1.0, seed=31)
    check_prefill(spec, label=f"bf16 dk={dk} dv={dv}")


@pytest.mark.parametrize("dk,dv,chunk", [(32, 32, 64), (64, 64, 64), (64, 32, 16), (128, 128, 16),
                                         (32, 128, 16), (128, 128, 64), (128, 64, 64), (64, 128, 64),
                                         (128, 32, 64)])
def test_fp32_shapes(dk, dv, chunk):
    """fp32 at the 1e-4 gate; chunk 64 with dk or dv = 128 takes the
    intra-chunk kernel's compact LDS placement."""
    spec = Spec(H=2, dk=dk, dv=dv, T=150, B=2, dtype="fp32", chunk=chunk, h0_std=1.0, g_mode="slow",
                seed=32)
    check_prefill(spec, label=f"fp32 dk={dk} dv={dv}")


@pytest.mark.parametrize("T", [1, 17, 33, 64, 128, 130, 192, 300, 384])
@pytest.mark.parametrize("B,H", [(1, 3), (2, 4)])
def test_bf16_chunk_counts(T, B, H):
    """d = 128, chunk 64 (the loader-fed state chain): 1 to 6 chunks per
    sequence, full and ragged last chunks (down to one token), so the chain's staging runs its
    prologue alone, its three-chunk groups and both tail lengths; B * H = 3
    and 8 chains take the two workgroup-to-chain mappings.  Slow decay and
    h0 ~ N(0, 1), so the carried state matters in every chunk."""
    spec = Spec(H=H, dk=128, dv=128, T=T, B=B, dtype="bf16", chunk=64, h0_std=1.0, g_mode="slow",
                seed=35 + T)
    check_prefill(spec, label=f"bf16 T={T} B={B} H={H}")


@pytest.mark.parametrize("mode", ["config", "slow", "floor", "zero"])
def test_bf16_decay_modes(mode):
    spec = Spec(H=4, dk=128, dv=128, T=1000, dtype="bf16", chunk=64, h0_std=1.0, g_mode=mode, seed=33)
    check_prefill(spec, label=f"bf16 g={mode}")


def test_state_isolation():
    """v = 0 and slow decay: o and the final state come only from h0 carried
    through every chunk."""
    spec = Spec(H=4, dk=128, dv=128, T=1000, dtype="bf16", chunk=64, h0_std=1.0, g_mode="slow",
                v_zero=True, seed=34)
    check_prefill(spec, label="state isolation")


def test_varlen_packed():
    """Packed sequences with empty, one-token and ragged lengths, per-sequence
    initial states and final states."""
    spec = Spec(H=3, dk=128, dv=128, seqlens=(37, 0, 64, 129, 1, 200, 16), dtype="bf16", chunk=64,
                h0_std=1.0, g_mode="slow", seed=35)
    check_prefill(spec, label="varlen")


def test_varlen_fp32_chunk16():
    spec = Spec(H=2, dk=32, dv=64, seqlens=(5, 33, 0, 16, 70), dtype="fp32", chunk=16, h0_std=1.0,
                g_mode="slow", seed=36)
    check_prefill(spec, label="varlen fp32")


def test_no_initial_state_and_no_final_state():
    spec = Spec(H=2, dk=64, dv=64, T=100, dtype="bf16", chunk=64, seed=37)
    x = workloads.make_prefill(spec)
    assert x["h0"] is None
    o, _ = gpu_prefill(x, 64, output_final_state=False)
    o_ref, _ = oracle_prefill(x)
    assert rel_l2(to_np64(o).reshape(o_ref.shape), o_ref) <= TOL_BF16


def test_resume_split():
    """prefill(T) == prefill(T1) then prefill(T - T1, h0 = ht_1), with the
    resumed call writing ht in place over h0."""
    import gated_delta_rule_97_amd as kda
    spec = Spec(H=4, dk=128, dv=128, T=700, dtype="bf16", chunk=64, h0_std=1.0, g_mode="slow", seed=38)
    x = workloads.make_prefill(spec)
    d = {k: (v.cuda() if v is not None else None) for k, v in x.items()}
    o_full, ht_full = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"])
    T1 = 300
    sl = lambda t, a, b: t[:, a:b].contiguous()
    o1, ht1 = kda.chunk_prefill(sl(d["q"], 0, T1), sl(d["k"], 0, T1), sl(d["v"], 0, T1),
                                sl(d["g"], 0, T1), sl(d["beta"], 0, T1), d["h0"])
    o2, ht2 = kda.chunk_prefill(sl(d["q"], T1, 700), sl(d["k"], T1, 700), sl(d["v"], T1, 700),
                                sl(d["g"], T1, 700), sl(d["beta"], T1, 700), ht1, ht=ht1)
    torch.cuda.synchronize()
    assert ht2.data_ptr() == ht1.data_ptr()
    o_ref, ht_ref = oracle_prefill(x)
    o_cat = torch.cat([o1, o2], dim=1)
    assert rel_l2(to_np64(o_cat).reshape(o_ref.shape), o_ref) <= TOL_BF16
    assert rel_l2(to_np64(ht2), ht_ref) <= TOL_BF16
    assert rel_l2(to_np64(o_cat), to_np64(o_full)) <= TOL_BF16


def test_chunk_size_invariance():
    spec = Spec(H=2, dk=128, dv=128, T=512, dtype="bf16", h0_std=1.0, g_mode="slow", seed=39)
    x = workloads.make_prefill(spec)
    o16, h16 = gpu_prefill(x, 16)
    o64, h64 = gpu_prefill(x, 64)
    assert rel_l2(to_np64(o16), to_np64(o64)) <= TOL_BF16
    assert rel_l2(to_np64(h16), to_np64(h64)) <= TOL_BF16


def test_prefill_equals_decode_steps():
    """A prefill over T tokens equals T decode steps on the same state."""
    import gated_delta_rule_97_amd as kda
    spec = Spec(H=4, dk=128, dv=64, T=40, dtype="bf16", chunk=16, h0_std=1.0, g_mode="slow", seed=40)
    x = workloads.make_prefill(spec)
    d = {k: (v.cuda() if v is not None else None) for k, v in x.items()}
    o, ht = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], chunk_size=16)
    state = d["h0"].clone()
    outs = []
    for t in range(40):
        outs.append(kda.decode_step(d["q"][:, t].contiguous(), d["k"][:, t].contiguous(),
                                    d["v"][:, t].contiguous(), d["g"][:, t].contiguous(),
                                    d["beta"][:, t].contiguous(), state))
    torch.cuda.synchronize()
    od = torch.stack(outs, dim=1)
    assert rel_l2(to_np64(od), to_np64(o)) <= TOL_BF16
    assert rel_l2(to_np64(state), to_np64(ht)) <= TOL_BF16


def test_fp32_chunk64_d128_packed_and_decay_floor():
    """fp32, d = 128, chunk 64 on packed sequences (empty, one-token and
    ragged) and at the decay bound itself (g = -5: the e^80 column operand)."""
    spec = Spec(H=2, dk=128, dv=128, seqlens=(70, 0, 1, 129, 64), dtype="fp32", chunk=64, h0_std=1.0,
                g_mode="slow", seed=42)
    check_prefill(spec, label="fp32 d128 chunk 64 packed")
    spec = Spec(H=2, dk=128, dv=128, T=333, dtype="fp32", chunk=64, h0_std=1.0, g_mode="floor", seed=43)
    check_prefill(spec, label="fp32 d128 chunk 64 g=-5")
