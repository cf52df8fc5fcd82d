"""Windows of the prefill: groups of whole sequences and chunk windows (needs a GPU).

A fixed-length bf16 batch at d = 128, chunk 64 whose hand-off between the
two passes passes 192 MiB runs as (intra-chunk pass, state pass) windows of
about 160 MiB, so that the state pass reads a hand-off the last-level cache
still holds: groups of whole sequences, or windows over the chunks of each
sequence with the state carried from one to the next in the workspace.  Windows change no arithmetic: the chain
takes the same products in the same order and the carried state is the
fp32 state itself, so o, the final state and the checkpoints must be
bit-identical to the one-pass chain (KDA_FLAG_NO_WINDOWS).  The windowed
headline's oracle parity is in test_gpu_full_size.py.

Page: the orkas.ai "Kimi K3 architecture" post, section on the serving
stack (the state updates serially, chunk after chunk).
"""
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


def _run(kda, x, T, **kw):
    return kda.chunk_prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], None, chunk_size=64, **kw)


def _intra_launches(kda, f):
    kda.kda_profile_start(64)
    out = f()
    torch.cuda.synchronize()
    kt = kda.kda_profile_stop()
    return kt["kda_intra"][0], out


# (B, T, H, windows): chunk windows of one sequence (2, ragged 2, 3), one
# sequence per window (2, ragged 2, 3), groups of four and two sequences,
# and two chunk windows in each of four sequences
@pytest.mark.parametrize("B,T,H,nwin", [(1, 8192, 32, 2), (1, 8152, 32, 2), (1, 12288, 32, 3), (2, 4096, 32, 2),
                                        (2, 4100, 32, 2), (3, 2752, 32, 3), (6, 1024, 32, 2), (4, 8192, 32, 8)])
def test_windows_equal_the_one_pass_chain(B, T, H, nwin):
    import gated_delta_rule_97_amd as kda
    spec = workloads.PREFILL_H32_T8K.replace(B=B, T=T, H=H, g_mode="slow", h0_std=1.0, seed=201)
    x = workloads.make_prefill(spec, device="cuda")
    print(f"[windows] B={B} T={T} H={H}", flush=True)
    n, (o, ht) = _intra_launches(kda, lambda: _run(kda, x, T))
    assert n == nwin, f"expected {nwin} windows, got {n} intra-chunk launches"
    n1, (o1, ht1) = _intra_launches(kda, lambda: _run(kda, x, T, flags=kda.KDA_FLAG_NO_WINDOWS))
    assert n1 == 1
    assert torch.equal(o, o1)
    assert torch.equal(ht, ht1)
    assert torch.isfinite(o.float()).all() and torch.isfinite(ht).all()
    # checkpoints every 512 tokens: the windows write them at the same
    # sequence positions
    n2, (o2, ht2, ck2) = _intra_launches(kda, lambda: _run(kda, x, T, ckpt_stride=512))
    n3, (o3, ht3, ck3) = _intra_launches(kda, lambda: _run(kda, x, T, ckpt_stride=512, flags=kda.KDA_FLAG_NO_WINDOWS))
    assert (n2, n3) == (nwin, 1)
    assert torch.equal(o2, o) and torch.equal(ht2, ht)
    assert torch.equal(ck2, ck3) and torch.equal(o3, o) and torch.equal(ht3, ht)


def test_windows_in_place_no_initial_and_no_final_state():
    import gated_delta_rule_97_amd as kda
    spec = workloads.PREFILL_H32_T8K.replace(g_mode="slow", h0_std=1.0, seed=202)
    x = workloads.make_prefill(spec, device="cuda")
    o, ht = _run(kda, x, 8192)
    # ht == h0: the first window reads h0 and hands its state on through the
    # carry; only the last window writes ht
    st = x["h0"].clone()
    o2, ht2 = kda.chunk_prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], st, None, chunk_size=64, ht=st)
    torch.cuda.synchronize()
    assert ht2.data_ptr() == st.data_ptr()
    assert torch.equal(o2, o) and torch.equal(st, ht)
    # no final state: the carry still hands the state from window to window
    o3, ht3 = kda.chunk_prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], None, chunk_size=64,
                                output_final_state=False)
    torch.cuda.synchronize()
    assert ht3 is None and torch.equal(o3, o)
    # no initial state: windowed against the one-pass chain
    oz, hz = kda.chunk_prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], None, None, chunk_size=64)
    oz1, hz1 = kda.chunk_prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], None, None, chunk_size=64,
                                 flags=kda.KDA_FLAG_NO_WINDOWS)
    torch.cuda.synchronize()
    assert torch.equal(oz, oz1) and torch.equal(hz, hz1)
