"""Error paths and non-finite inputs (needs a GPU).

* KDA_FLAG_CHECK_DECAY on the prefill: g outside [-5, 0] (or NaN) gives
  KDA_ERR_DECAY_BOUND and a malformed cu_seqlens gives KDA_ERR_SHAPE, with
  nothing launched (o and ht keep their previous bytes); inputs that pass
  give exactly the unchecked call's results.  The bound is the method's
  precondition (orkas.ai "Kimi K3 architecture", section on the lower bound
  that removed a GPU code path: every per-step log-decay is at least -5).
* A NaN input is not hidden and does not spread beyond what it feeds: a NaN
  key channel poisons its (sequence, head) from the NaN on, a NaN value
  channel only that value column of it (every product is column-local in
  v); on the GPU the poisoning starts at the NaN's 64-token chunk (the
  chunk's products mix all of its tokens, 0 * NaN included).  Every other
  head and sequence is unaffected and still matches the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import TOL_BF16, rel_l2
from kda_cases import oracle_prefill, to_np64

pytestmark = pytest.mark.gpu

Spec = workloads.PrefillSpec


def _dev(x):
    return {key: (val.cuda() if val is not None else None) for key, val in x.items()}


@pytest.mark.parametrize("packed", [False, True])
def test_prefill_check_flag(packed):
    import gated_delta_rule_97_amd as kda
    if packed:
        spec = Spec(H=2, dk=128, dv=128, seqlens=(70, 0, 129), dtype="bf16", chunk=64, h0_std=1.0, seed=111)
    else:
        spec = Spec(H=2, dk=128, dv=128, T=150, B=2, dtype="bf16", chunk=64, h0_std=1.0, seed=111)
    d = _dev(workloads.make_prefill(spec))
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"])
    o_plain, ht_plain = kda.chunk_prefill(*args)
    o_chk, ht_chk = kda.chunk_prefill(*args, flags=kda.KDA_FLAG_CHECK_DECAY)
    torch.cuda.synchronize()
    assert torch.equal(o_plain, o_chk) and torch.equal(ht_plain, ht_chk), "a passing check changes nothing"

    def rejected(status, g=None, cu=None):
        o = torch.full_like(o_plain, 7.0)
        ht = torch.full_like(ht_plain, -3.0)
        a = list(args)
        if g is not None:
            a[3] = g
        if cu is not None:
            a[6] = cu
        with pytest.raises(kda.KdaError) as e:
            kda.chunk_prefill(*a, o=o, ht=ht, flags=kda.KDA_FLAG_CHECK_DECAY)
        assert e.value.status == status, kda.kda_status_string(e.value.status)
        torch.cuda.synchronize()
        assert bool((o == 7.0).all()) and bool((ht == -3.0).all()), "a rejected call must launch nothing"

    for bad in (-5.5, 0.25, float("nan"), float("-inf")):
        g = d["g"].clone()
        g[0, 37, 1, 5] = bad
        rejected(kda.KDA_ERR_DECAY_BOUND, g=g)
    g = d["g"].clone()
    g[0, 0, 0, 0] = -5.0  # the bound itself is allowed
    o_b, _ = kda.chunk_prefill(*args[:3], g, *args[4:], flags=kda.KDA_FLAG_CHECK_DECAY)
    torch.cuda.synchronize()
    assert torch.isfinite(o_b.float()).all()
    if packed:
        T = d["q"].shape[1]
        for cu in ([0, 70, 60, T], [0, 70, 70, T - 1], [1, 70, 70, T]):
            rejected(kda.KDA_ERR_SHAPE, cu=torch.tensor(cu, dtype=torch.int32, device="cuda"))


def _nan_case(segmented, which):
    """A prefill with one NaN input element at (sequence n, token t, head h,
    channel j); returns (inputs, GPU o, GPU ht, oracle o, oracle ht, n, t, h,
    j) with o as [B, T, H, dv]."""
    import gated_delta_rule_97_amd as kda
    T = 128 * 64 + 37 if segmented else 300
    H = 1 if segmented else 3
    spec = Spec(H=H, dk=128, dv=128, T=T, B=2, dtype="bf16", chunk=64, h0_std=1.0, g_mode="slow", seed=112)
    x = workloads.make_prefill(spec)
    n, h, t, j = 1, H - 1, 2 * 64 + 21, 7
    x[which][n, t, h, j] = float("nan")
    d = _dev(x)
    kda.kda_profile_start(64)
    o, ht = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], chunk_size=64)
    kt = kda.kda_profile_stop()
    torch.cuda.synchronize()
    assert ("kda_seg_scan" in kt) == segmented
    o_ref, ht_ref = oracle_prefill(x)
    return x, to_np64(o), to_np64(ht), o_ref.reshape(o.shape), ht_ref, n, t, h, j


def _other_heads_clean(on, hn, o_ref, ht_ref, n, h):
    B, H = on.shape[0], on.shape[2]
    for m in range(B):
        for i in range(H):
            if (m, i) != (n, h):
                assert np.all(np.isfinite(on[m, :, i])) and np.all(np.isfinite(hn[m, i])), (m, i)
                assert rel_l2(on[m, :, i], o_ref[m, :, i]) <= TOL_BF16, (m, i)
                assert rel_l2(hn[m, i], ht_ref[m, i]) <= TOL_BF16, (m, i)


@pytest.mark.parametrize("segmented", [False, True])
def test_prefill_nan_in_k_poisons_only_its_head(segmented):
    """A NaN key channel enters every column through k^T S: the head's state
    and every output from the NaN on are NaN (from its chunk's start on the
    GPU), every other head and sequence is untouched."""
    x, on, hn, o_ref, ht_ref, n, t, h, j = _nan_case(segmented, "k")
    c0 = (t // 64) * 64
    assert np.all(np.isnan(on[n, t:, h])), "every output of the head from the NaN on is NaN"
    assert np.all(np.isnan(hn[n, h])), "the head's final state is NaN"
    assert np.all(np.isnan(o_ref[n, t:, h])) and np.all(np.isfinite(o_ref[n, :t, h]))  # the oracle agrees
    before = on[n, :c0, h]
    assert np.all(np.isfinite(before)) and rel_l2(before, o_ref[n, :c0, h]) <= TOL_BF16
    _other_heads_clean(on, hn, o_ref, ht_ref, n, h)


@pytest.mark.parametrize("segmented", [False, True])
def test_prefill_nan_in_v_poisons_only_its_value_column(segmented):
    """A NaN value channel j reaches only column j of the head's state (every
    product is column-local in v): o[.., j] from the NaN on (from its chunk's
    start on the GPU) and ht[.., j] are NaN, every other column, head and
    sequence still matches the oracle."""
    x, on, hn, o_ref, ht_ref, n, t, h, j = _nan_case(segmented, "v")
    c0 = (t // 64) * 64
    cols = np.arange(on.shape[-1]) != j
    assert np.all(np.isnan(on[n, t:, h, j])) and np.all(np.isnan(hn[n, h, :, j]))
    assert np.all(np.isnan(o_ref[n, t:, h, j])) and np.all(np.isfinite(o_ref[n, :, h][:, cols]))
    assert np.all(np.isfinite(on[n, :, h][:, cols])) and np.all(np.isfinite(hn[n, h][:, cols]))
    assert rel_l2(on[n, :, h][:, cols], o_ref[n, :, h][:, cols]) <= TOL_BF16
    assert rel_l2(hn[n, h][:, cols], ht_ref[n, h][:, cols]) <= TOL_BF16
    assert np.all(np.isfinite(on[n, :c0, h, j])) and rel_l2(on[n, :c0, h, j], o_ref[n, :c0, h, j]) <= TOL_BF16
    _other_heads_clean(on, hn, o_ref, ht_ref, n, h)


def test_decode_nan_stays_in_its_head():
    import gated_delta_rule_97_amd as kda
    spec = workloads.DecodeSpec(N=6, H=3, dk=128, dv=128, steps=2, dtype="bf16", state_std=1.0, g_mode="slow",
                                seed=113)
    s0 = workloads.make_decode_state(spec)
    ref = s0.numpy().astype(np.float64)
    state = s0.cuda()
    for step in range(2):
        x = workloads.make_decode_step(spec, step)
        if step == 0:
            x["k"][4, 1, 9] = float("nan")
        o = kda.decode_step(*(x[key].cuda() for key in ("q", "k", "v", "g", "beta")), state)
        o_ref = oracle.decode_step(*(workloads.to_numpy_f32(x[key]) for key in ("q", "k", "v", "g", "beta")), ref)
        torch.cuda.synchronize()
        on = o.double().cpu().numpy()
        assert np.all(np.isnan(on[4, 1])), f"step {step}: the poisoned head's output is NaN"
        mask = np.ones((6, 3), dtype=bool)
        mask[4, 1] = False
        assert np.all(np.isfinite(on[mask]))
        assert rel_l2(on[mask], o_ref[mask]) <= TOL_BF16
    sn = state.double().cpu().numpy()
    assert np.all(np.isnan(sn[4, 1]))
    mask = np.ones((6, 3), dtype=bool)
    mask[4, 1] = False
    assert np.all(np.isfinite(sn[mask])) and rel_l2(sn[mask], ref[mask]) <= TOL_BF16
