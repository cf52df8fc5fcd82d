"""The prefill workloads at their full sizes against the fp64 oracle (needs a
GPU), every output and every final state, with the per-(sequence, head)
gates as well as the whole-tensor ones:

* H=32, T=8192, d=128, bf16, chunk 64: the configs' own decay with
  h0 ~ N(0, 0.02), then slow decay with h0 ~ N(0, 1) and state isolation
  (v = 0, no decay), where o and the final state come only from the
  carried state;
* 64 packed sequences of U[256, 4096] tokens, H=16, per-sequence h0, every
  sequence;
* 1M tokens x 8 heads: the oracle streams the sequence in token slices,
  resuming each slice from its own fp64 final state (a resume is exact:
  pin P12), and accumulates the error norms of every head as it goes; the
  segmented chain (the default at this size) and the single chain are both
  checked.

Pages: the poyo.ai "Kimi K3 architecture" hub, section on how K3 reaches a
1M-token context; the orkas.ai "Kimi K3 architecture" post, section on the
serving stack (prefix reuse across requests).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import TOL_BF16, rel_l2_per_state, worst
from kda_cases import check_prefill, to_np64

pytestmark = pytest.mark.gpu


def test_headline_config_full_size():
    """B=1, H=32, T=8192, d=128, bf16, chunk 64, h0 ~ N(0, 0.02)."""
    check_prefill(workloads.PREFILL_H32_T8K, label="headline prefill H=32 T=8192")


def test_headline_shape_slow_decay():
    """The headline shape with long memory: a broken inter-chunk carry moves
    o by about half its norm here (against ~2% at the configs' decay)."""
    spec = workloads.PREFILL_H32_T8K.replace(g_mode="slow", h0_std=1.0, seed=101)
    check_prefill(spec, label="headline shape, slow decay, h0 N(0,1)")


def test_headline_shape_state_isolation():
    """v = 0: o and the final state come only from h0 carried through all
    128 chunks of every head.  With no decay, so that the final state stays
    inside fp32's range: the erase steps alone shrink h0's share to about
    1e-10 over 8192 tokens, while slow decay would take it to ~e^-164, which
    underflows (the oracle's fp64 keeps it, the GPU's fp32 state cannot).

    The whole tensors keep the 2e-2 gate.  Each head's final state is gated
    at a stated 3e-2: in this pure carry every chunk rounds the carried
    state and U to bf16 for its products (relative 2^-9 each) and nothing
    decays the earlier roundings away, so they add up like a random walk
    over the 128 chunks, about sqrt(128) * 2^-9 ~ 2e-2, and single heads
    scatter around that (measured: whole 1.7e-2, worst head 2.1e-2)."""
    spec = workloads.PREFILL_H32_T8K.replace(g_mode="zero", h0_std=1.0, v_zero=True, seed=102)
    check_prefill(spec, label="headline shape, state isolation", block_tol=3e-2)


@pytest.mark.parametrize("mode,h0_std", [("config", 0.02), ("slow", 1.0)])
def test_varlen_full_size(mode, h0_std):
    """All 64 packed sequences, H=16, d=128, bf16, chunk 64, per-sequence h0."""
    spec = workloads.VARLEN_64_SEQS.replace(g_mode=mode, h0_std=h0_std)
    check_prefill(spec, label=f"varlen 64 sequences T={spec.total_tokens} g={mode}")


def _stream_oracle(x, outs, slice_tokens):
    """fp64 oracle over one long sequence, slice by slice, resuming from its
    own final state; accumulates per-head squared errors of every GPU output
    in ``outs`` ({name: o [1, T, H, dv] on the device}).  Returns ({name:
    (err2 [H], ref2 [H])}, final state [1, H, dk, dv])."""
    T, H = x["q"].shape[1], x["q"].shape[2]
    S = None if x["h0"] is None else x["h0"].cpu().numpy().astype(np.float64)
    acc = {name: (np.zeros(H), np.zeros(H)) for name in outs}
    for a in range(0, T, slice_tokens):
        b = min(T, a + slice_tokens)
        f = lambda t: t[0, a:b].float().cpu().numpy()
        o_ref, S = oracle.prefill(f(x["q"]), f(x["k"]), f(x["v"]), f(x["g"]), f(x["beta"]), S)
        ref2 = np.sum(o_ref ** 2, axis=(0, 2))
        for name, o in outs.items():
            og = o[0, a:b].double().cpu().numpy()
            e2, r2 = acc[name]
            e2 += np.sum((og - o_ref) ** 2, axis=(0, 2))
            r2 += ref2
        print(f"[parity]   oracle tokens {a}..{b}", flush=True)
    return acc, S


@pytest.mark.parametrize("mode", ["config", "slow"])
def test_long_context_full_size(mode):
    """1M tokens x 8 heads, d=128, bf16, chunk 64: every output and the final
    state of every head against the oracle, for the segmented chain and for
    the single chain per head."""
    import gated_delta_rule_97_amd as kda
    spec = workloads.LONG_CONTEXT_1M.replace(g_mode=mode)
    dev = torch.device("cuda")
    print(f"[parity] 1M tokens g={mode}: generating on the GPU", flush=True)
    x = workloads.make_prefill(spec, device=dev)
    outs, states = {}, {}
    for name, flags in (("segmented", 0), ("single chain", kda.KDA_FLAG_NO_SEGMENTS)):
        o, ht = kda.chunk_prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], chunk_size=64, flags=flags)
        torch.cuda.synchronize()
        assert torch.isfinite(ht).all() and torch.isfinite(o.float()).all(), name
        outs[name], states[name] = o, ht
    acc, S = _stream_oracle(x, outs, 1 << 16)
    for name in outs:
        e2, r2 = acc[name]
        eo = float(np.sqrt(e2.sum() / r2.sum()))
        wo = float(np.max(np.sqrt(e2 / r2)))
        hs = to_np64(states[name])
        per_h = rel_l2_per_state(hs, S)
        eh = float(np.linalg.norm(hs - S) / np.linalg.norm(S))
        print(f"[parity]   1M {name} g={mode}: rel-L2 o={eo:.3e} ht={eh:.3e}; worst head o={wo:.3e} "
              f"ht={worst(per_h):.3e}", flush=True)
        assert eo <= TOL_BF16 and wo <= TOL_BF16, name
        assert eh <= TOL_BF16 and worst(per_h) <= TOL_BF16, name
