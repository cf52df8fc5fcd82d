"""Seeded synthetic KDA workloads.

This module only draws inputs.  It holds none of the method's arithmetic, so
both the HIP path and the oracle may take their inputs from it.

Recipe (per (token, head) row, all in float32 before any cast):
  q, k ~ N(0, 1), then L2-normalised over the head dimension;
  v ~ N(0, 1);
  beta = sigmoid(N(0, 1));
  g (per channel, natural-log decay) by ``g_mode``:
      "config": -5 * sigmoid(N(0, 1))     (in (-5, 0): the per-step floor of
                                           the blog post's decay bound)
      "slow":   -5 * sigmoid(N(-6, 1))    (mean about -0.02: long memory)
      "floor":  -5 everywhere             (the bound reached exactly)
      "zero":   0 everywhere              (no decay)
  h0 ~ N(0, h0_std) when h0_std > 0, else no initial state;
  q/k/v are then cast to the compute dtype (bf16 with round-to-nearest-even,
  or kept float32).  g, beta, h0 stay float32.

Shapes follow the workloads of the Kimi K3 pages: head dimension 128,
contexts up to 1M tokens, many independent decode streams.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

G_MODES = ("config", "slow", "floor", "zero")


@dataclass(frozen=True)
class PrefillSpec:
    H: int
    dk: int
    dv: int
    T: int = 0                       # tokens per sequence (fixed-length batch)
    B: int = 1                       # fixed-length sequences
    seqlens: Optional[tuple] = None  # packed variable-length sequences (B must be 1)
    dtype: str = "bf16"              # "bf16" or "fp32" for q, k, v, o
    chunk: int = 64
    g_mode: str = "config"
    h0_std: float = 0.0
    v_zero: bool = False
    seed: int = 0
    name: str = ""

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seqlens)) if self.seqlens is not None else self.B * self.T

    @property
    def num_seqs(self) -> int:
        return len(self.seqlens) if self.seqlens is not None else self.B

    def replace(self, **kw) -> "PrefillSpec":
        return dataclasses.replace(self, **kw)


@dataclass(frozen=True)
class DecodeSpec:
    N: int
    H: int
    dk: int
    dv: int
    steps: int
    dtype: str = "bf16"
    g_mode: str = "config"
    state_std: float = 0.02
    seed: int = 4
    name: str = ""

    def replace(self, **kw) -> "DecodeSpec":
        return dataclasses.replace(self, **kw)


def varlen_lengths(n: int, lo: int, hi: int, seed: int) -> tuple:
    """n integer lengths uniform in [lo, hi] (inclusive), seeded."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return tuple(int(x) for x in rng.integers(lo, hi + 1, size=n))


# The five workloads: a tiny fp32 case, the headline prefill, packed
# variable-length prefill with per-sequence initial states, 1M-token prefill,
# and 256-stream decode.
TINY_FP32 = PrefillSpec(H=2, dk=32, dv=32, T=64, dtype="fp32", chunk=16, seed=0,
                        name="tiny fp32 prefill H=2 T=64 d=32 chunk=16")
PREFILL_H32_T8K = PrefillSpec(H=32, dk=128, dv=128, T=8192, dtype="bf16", chunk=64,
                              h0_std=0.02, seed=1,
                              name="prefill B=1 H=32 T=8192 d=128 bf16")
VARLEN_64_SEQS = PrefillSpec(H=16, dk=128, dv=128, seqlens=varlen_lengths(64, 256, 4096, 2),
                             dtype="bf16", chunk=64, h0_std=0.02, seed=2,
                             name="varlen prefill 64 seqs U[256,4096] H=16 d=128 bf16")
LONG_CONTEXT_1M = PrefillSpec(H=8, dk=128, dv=128, T=1 << 20, dtype="bf16", chunk=64, seed=3,
                              name="long-context prefill B=1 H=8 T=1048576 d=128 bf16")
PREFILL_WORKLOADS = (TINY_FP32, PREFILL_H32_T8K, VARLEN_64_SEQS, LONG_CONTEXT_1M)
DECODE = DecodeSpec(N=256, H=32, dk=128, dv=128, steps=128, dtype="bf16",
                    state_std=0.02, seed=4,
                    name="decode N=256 H=32 d=128 bf16, 128 steps")


def _torch_dtype(name: str):
    return {"bf16": torch.bfloat16, "fp32": torch.float32}[name]


def _gen(seed: int, device) -> torch.Generator:
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    return gen


def _unit_rows(shape, gen, device):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)


def _decay(shape, mode, gen, device):
    if mode == "config":
        z = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        return -5.0 * torch.sigmoid(z)
    if mode == "slow":
        z = torch.randn(shape, generator=gen, device=device, dtype=torch.float32) - 6.0
        return -5.0 * torch.sigmoid(z)
    if mode == "floor":
        return torch.full(shape, -5.0, device=device, dtype=torch.float32)
    if mode == "zero":
        return torch.zeros(shape, device=device, dtype=torch.float32)
    raise ValueError(f"unknown g_mode {mode!r}")


def make_prefill(spec: PrefillSpec, device="cpu") -> dict:
    """Draw one prefill batch.  Returns a dict of torch tensors on ``device``:
    q, k [B, T, H, dk]; v [B, T, H, dv] (compute dtype); g [B, T, H, dk],
    beta [B, T, H] (float32); h0 [N, H, dk, dv] float32 or None;
    cu_seqlens int32 [N+1] or None (packed: B = 1, T = sum of lengths)."""
    if spec.g_mode not in G_MODES:
        raise ValueError(spec.g_mode)
    gen = _gen(spec.seed, device)
    if spec.seqlens is not None:
        if spec.B != 1:
            raise ValueError("packed sequences need B == 1")
        B, T = 1, spec.total_tokens
        cu = torch.tensor(np.concatenate([[0], np.cumsum(spec.seqlens)]),
                          dtype=torch.int32, device=device)
    else:
        B, T = spec.B, spec.T
        cu = None
    H, dk, dv = spec.H, spec.dk, spec.dv
    dt = _torch_dtype(spec.dtype)
    q = _unit_rows((B, T, H, dk), gen, device).to(dt)
    k = _unit_rows((B, T, H, dk), gen, device).to(dt)
    v = torch.randn((B, T, H, dv), generator=gen, device=device, dtype=torch.float32)
    if spec.v_zero:
        v.zero_()
    v = v.to(dt)
    beta = torch.sigmoid(torch.randn((B, T, H), generator=gen, device=device,
                                     dtype=torch.float32))
    g = _decay((B, T, H, dk), spec.g_mode, gen, device)
    h0 = None
    if spec.h0_std > 0:
        h0 = spec.h0_std * torch.randn((spec.num_seqs, H, dk, dv), generator=gen,
                                       device=device, dtype=torch.float32)
    return {"q": q, "k": k, "v": v, "g": g, "beta": beta, "h0": h0,
            "cu_seqlens": cu}


def make_decode_state(spec: DecodeSpec, device="cpu") -> torch.Tensor:
    """Initial fp32 state [N, H, dk, dv] ~ N(0, state_std)."""
    gen = _gen(spec.seed, device)
    return spec.state_std * torch.randn((spec.N, spec.H, spec.dk, spec.dv),
                                        generator=gen, device=device,
                                        dtype=torch.float32)


def make_decode_drafts(spec: DecodeSpec, K: int, first_step: int = 0, device="cpu") -> dict:
    """K consecutive decode steps stacked as draft tokens: q, k [N, K, H, dk];
    v [N, K, H, dv]; g [N, K, H, dk]; beta [N, K, H] (token t is step
    first_step + t of ``make_decode_step``)."""
    steps = [make_decode_step(spec, first_step + t, device) for t in range(K)]
    return {key: torch.stack([st[key] for st in steps], dim=1).contiguous() for key in steps[0]}


def make_decode_step(spec: DecodeSpec, step: int, device="cpu") -> dict:
    """Inputs of decode step ``step``: q, k [N, H, dk]; v [N, H, dv] (compute
    dtype); g [N, H, dk], beta [N, H] (float32)."""
    gen = _gen(spec.seed * 1000003 + 7919 * (step + 1), device)
    N, H, dk, dv = spec.N, spec.H, spec.dk, spec.dv
    dt = _torch_dtype(spec.dtype)
    q = _unit_rows((N, H, dk), gen, device).to(dt)
    k = _unit_rows((N, H, dk), gen, device).to(dt)
    v = torch.randn((N, H, dv), generator=gen, device=device, dtype=torch.float32).to(dt)
    beta = torch.sigmoid(torch.randn((N, H), generator=gen, device=device,
                                     dtype=torch.float32))
    g = _decay((N, H, dk), spec.g_mode, gen, device)
    return {"q": q, "k": k, "v": v, "g": g, "beta": beta}


def to_numpy_f32(x: Optional[torch.Tensor]):
    """Exact float32 host copy (bf16 values are exactly representable)."""
    if x is None:
        return None
    return x.detach().to("cpu", torch.float32).numpy()
