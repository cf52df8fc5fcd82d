"""The seeded generators: determinism, shapes, dtypes and distributions."""
import numpy as np
import torch

import workloads


def test_workload_shapes():
    c1 = workloads.PREFILL_H32_T8K
    assert (c1.H, c1.dk, c1.dv, c1.T, c1.chunk) == (32, 128, 128, 8192, 64)
    c2 = workloads.VARLEN_64_SEQS
    assert len(c2.seqlens) == 64 and min(c2.seqlens) >= 256 and max(c2.seqlens) <= 4096
    assert workloads.LONG_CONTEXT_1M.T == 1 << 20
    d = workloads.DECODE
    assert (d.N, d.H, d.dk, d.steps) == (256, 32, 128, 128)


def test_deterministic_and_recipe():
    spec = workloads.PrefillSpec(H=4, dk=32, dv=16, T=200, h0_std=0.02, seed=9)
    a = workloads.make_prefill(spec)
    b = workloads.make_prefill(spec)
    for key in ("q", "k", "v", "g", "beta", "h0"):
        assert torch.equal(a[key], b[key])
    assert a["q"].dtype == torch.bfloat16 and a["g"].dtype == torch.float32
    n = torch.linalg.vector_norm(a["k"].float(), dim=-1)
    assert torch.allclose(n, torch.ones_like(n), atol=1e-2)
    assert float(a["g"].min()) >= -5.0 and float(a["g"].max()) < 0.0
    assert 0.0 < float(a["beta"].min()) and float(a["beta"].max()) < 1.0
    assert abs(float(a["h0"].std()) - 0.02) < 0.002
    c = workloads.make_prefill(spec.replace(seed=10))
    assert not torch.equal(a["q"], c["q"])


def test_varlen_and_modes():
    spec = workloads.PrefillSpec(H=2, dk=16, dv=16, seqlens=(3, 0, 50), g_mode="slow")
    x = workloads.make_prefill(spec)
    assert x["q"].shape == (1, 53, 2, 16)
    assert x["cu_seqlens"].tolist() == [0, 3, 3, 53]
    assert float(x["g"].mean()) > -0.1
    x = workloads.make_prefill(spec.replace(g_mode="floor", v_zero=True))
    assert torch.all(x["g"] == -5.0) and torch.all(x["v"] == 0)


def test_decode_inputs():
    spec = workloads.DecodeSpec(N=3, H=2, dk=16, dv=8, steps=2)
    s = workloads.make_decode_state(spec)
    assert s.shape == (3, 2, 16, 8) and s.dtype == torch.float32
    a = workloads.make_decode_step(spec, 0)
    b = workloads.make_decode_step(spec, 1)
    assert a["q"].shape == (3, 2, 16) and not torch.equal(a["q"], b["q"])
    assert np.array_equal(workloads.to_numpy_f32(a["q"]), a["q"].float().numpy())
