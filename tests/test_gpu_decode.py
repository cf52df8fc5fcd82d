"""Parity of the HIP decode step against the fp64 oracle (needs a GPU)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import TOL_BF16, TOL_FP32, rel_l2

pytestmark = pytest.mark.gpu


def _np(t):
    return workloads.to_numpy_f32(t)


def _run(spec, steps):
    import gated_delta_rule_97_amd as kda
    state0 = workloads.make_decode_state(spec)
    ref_state = state0.numpy().astype(np.float64)
    state = state0.cuda()
    errs = []
    for s in range(steps):
        x = workloads.make_decode_step(spec, s)
        d = {k: v.cuda() for k, v in x.items()}
        o = kda.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state)
        o_ref = oracle.decode_step(_np(x["q"]), _np(x["k"]), _np(x["v"]), _np(x["g"]), _np(x["beta"]),
                                   ref_state)
        torch.cuda.synchronize()
        errs.append(rel_l2(o.double().cpu().numpy(), o_ref))
    es = rel_l2(state.double().cpu().numpy(), ref_state)
    return max(errs), es


@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_decode_small(dk, dv, dtype):
    spec = workloads.DecodeSpec(N=5, H=3, dk=dk, dv=dv, steps=4, dtype=dtype, state_std=1.0,
                                g_mode="slow", seed=41)
    eo, es = _run(spec, 4)
    tol = TOL_FP32 if dtype == "fp32" else TOL_BF16
    print(f"[decode] dk={dk} dv={dv} {dtype}: o {eo:.2e} state {es:.2e}", flush=True)
    assert eo <= tol and es <= tol


@pytest.mark.parametrize("mode", ["config", "floor", "zero"])
def test_decode_decay_modes(mode):
    """Decode under the configs' fast decay, the bound itself (g = -5 every
    step, the smallest kept fraction) and no decay at all, over enough steps
    that the state carries several tokens."""
    spec = workloads.DecodeSpec(N=7, H=4, dk=128, dv=128, steps=12, dtype="bf16", state_std=1.0,
                                g_mode=mode, seed=43)
    eo, es = _run(spec, 12)
    print(f"[decode] g={mode}: o {eo:.2e} state {es:.2e}", flush=True)
    assert np.isfinite(eo) and np.isfinite(es)
    assert eo <= TOL_BF16 and es <= TOL_BF16


def test_decode_single_sequence_head():
    """The smallest grid: one (sequence, head), fp32, every shape kernel."""
    for dk, dv in [(32, 32), (128, 128)]:
        spec = workloads.DecodeSpec(N=1, H=1, dk=dk, dv=dv, steps=3, dtype="fp32", state_std=1.0,
                                    g_mode="slow", seed=44)
        eo, es = _run(spec, 3)
        print(f"[decode] N=H=1 dk={dk} dv={dv}: o {eo:.2e} state {es:.2e}", flush=True)
        assert eo <= TOL_FP32 and es <= TOL_FP32


def test_decode_headline_batch_all_steps():
    """The 256-sequence x 32-head decode batch, all 128 consecutive in-place
    steps, every output of every step and the whole final state checked."""
    spec = workloads.DECODE
    eo, es = _run(spec, spec.steps)
    print(f"[decode] headline: o {eo:.2e} state {es:.2e}", flush=True)
    assert eo <= TOL_BF16 and es <= TOL_BF16


def test_decode_check_flag():
    import gated_delta_rule_97_amd as kda
    spec = workloads.DecodeSpec(N=2, H=2, dk=32, dv=32, steps=1, dtype="bf16")
    x = {k: v.cuda() for k, v in workloads.make_decode_step(spec, 0).items()}
    state = workloads.make_decode_state(spec).cuda()
    kda.decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], state, flags=kda.KDA_FLAG_CHECK_DECAY)
    x["g"][1, 1, 3] = -5.5
    before = state.clone()
    with pytest.raises(kda.KdaError) as e:
        kda.decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], state, flags=kda.KDA_FLAG_CHECK_DECAY)
    assert e.value.status == kda.KDA_ERR_DECAY_BOUND
    torch.cuda.synchronize()
    assert torch.equal(before, state), "a rejected call must not touch the state"
