"""Pins for the fp64 oracle: checks against closed forms, brute force and the
structural facts on the Kimi K3 pages, chosen so that a plausible mistake in
the oracle (a dropped term, a wrong sign or index, a transposed operand, the
wrong order of decay / erase / write / read) fails at least one of them.

All of these run on the CPU (no GPU marker).  ``PINS`` is a list of
functions taking a runner ``run(q, k, v, g, beta, h0, cu) -> (o, ht)`` over
packed [T, H, d] float64 arrays; the oracle must pass every pin, and each
planted mistake in ``test_pins_catch_planted_mistakes`` must fail one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from chunked_fp64 import chunked_prefill
from helpers import rel_l2

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _unit(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _f32(x):
    """Round to float32 so both oracle implementations see the same values."""
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def rand_case(seed, T, H, dk, dv, *, g_lo=-5.0, beta=None, h0_std=1.0):
    rng = _rng(seed)
    q = _f32(_unit(rng, (T, H, dk)))
    k = _f32(_unit(rng, (T, H, dk)))
    v = _f32(rng.standard_normal((T, H, dv)))
    g = _f32(rng.uniform(g_lo, 0.0, (T, H, dk)))
    b = _f32(rng.uniform(0.0, 1.0, (T, H)) if beta is None else np.full((T, H), beta))
    h0 = rng.standard_normal((1, H, dk, dv)) * h0_std if h0_std else None
    return q, k, v, g, b, h0


def run_c(q, k, v, g, beta, h0=None, cu=None):
    return oracle.prefill(q, k, v, g, beta, h0, cu)


def run_np(q, k, v, g, beta, h0=None, cu=None):
    return oracle.prefill_np(q, k, v, g, beta, h0, cu)


# ---------------------------------------------------------------- the pins

def pin_p2_bruteforce(run):
    """P2: explicit dk x dk transitions M_t = (I - b_t k_t k_t^T) Diag(e^{g_t});
    S_t = M_t...M_1 h0 + sum_s M_t...M_{s+1} b_s k_s v_s^T, o_t = S_t^T q_t,
    evaluated as unrolled matrix products for T <= 8 (dk != dv)."""
    T, H, dk, dv = 7, 2, 5, 3
    q, k, v, g, b, h0 = rand_case(11, T, H, dk, dv)
    o, ht = run(q, k, v, g, b, h0)
    for h in range(H):
        M = [(np.eye(dk) - b[t, h] * np.outer(k[t, h], k[t, h])) @ np.diag(np.exp(g[t, h]))
             for t in range(T)]
        for t in range(T):
            # M_t ... M_0 h0 + sum_s (M_t ... M_{s+1}) b_s k_s v_s^T
            St = np.eye(dk)
            for u in range(t, -1, -1):
                St = St @ M[u]
            St = St @ h0[0, h]
            for s in range(t + 1):
                Ps = np.eye(dk)
                for u in range(t, s, -1):
                    Ps = Ps @ M[u]
                St = St + Ps @ (b[s, h] * np.outer(k[s, h], v[s, h]))
            assert np.allclose(o[t, h], St.T @ q[t, h], rtol=1e-12, atol=1e-13), "P2 o"
            if t == T - 1:
                assert np.allclose(ht[0, h], St, rtol=1e-12, atol=1e-13), "P2 ht"


def pin_p3_beta_zero(run):
    """P3: beta = 0 leaves only the decay: S_t = Diag(e^{Gam_t}) h0 and
    o_t[j] = sum_c q_t[c] e^{Gam_t[c]} h0[c, j]."""
    T, H, dk, dv = 9, 2, 6, 4
    q, k, v, g, b, h0 = rand_case(12, T, H, dk, dv, g_lo=-1.0, beta=0.0)
    o, ht = run(q, k, v, g, b, h0)
    Gam = np.cumsum(g, axis=0)
    for h in range(H):
        for t in range(T):
            ref = np.array([sum(q[t, h, c] * math.exp(Gam[t, h, c]) * h0[0, h, c, j]
                                for c in range(dk)) for j in range(dv)])
            assert np.allclose(o[t, h], ref, rtol=1e-12, atol=1e-14), "P3 o"
        ref_ht = np.exp(Gam[-1, h])[:, None] * h0[0, h]
        assert np.allclose(ht[0, h], ref_ht, rtol=1e-12, atol=1e-14), "P3 ht"


def pin_p4_one_hot(run):
    """P4: one-hot keys k_t = e_{i_t} make the rows independent scalar EMAs:
    row i_t: S <- (1 - b_t) e^{g_t[i_t]} S + b_t v_t; other rows S <- e^{g_t[j]} S."""
    T, H, dk, dv = 12, 1, 4, 3
    rng = _rng(13)
    idx = rng.integers(0, dk, size=T)
    k = np.zeros((T, H, dk))
    k[np.arange(T), 0, idx] = 1.0
    q = _f32(rng.standard_normal((T, H, dk)))
    v = _f32(rng.standard_normal((T, H, dv)))
    g = _f32(rng.uniform(-2.0, 0.0, (T, H, dk)))
    b = _f32(rng.uniform(0.0, 1.0, (T, H)))
    h0 = rng.standard_normal((1, H, dk, dv))
    o, ht = run(q, k, v, g, b, h0)
    S = [list(h0[0, 0, i]) for i in range(dk)]
    for t in range(T):
        for i in range(dk):
            f = math.exp(g[t, 0, i])
            for j in range(dv):
                if i == idx[t]:
                    S[i][j] = (1.0 - b[t, 0]) * f * S[i][j] + b[t, 0] * v[t, 0, j]
                else:
                    S[i][j] = f * S[i][j]
        for j in range(dv):
            ref = sum(q[t, 0, i] * S[i][j] for i in range(dk))
            assert abs(o[t, 0, j] - ref) <= 1e-12 * (1 + abs(ref)), "P4 o"
    assert np.allclose(ht[0, 0], np.array(S), rtol=1e-12, atol=1e-14), "P4 ht"


def pin_p5_orthonormal(run):
    """P5: orthonormal keys, g = 0, zero start, T <= dk: the erase term
    vanishes and KDA is textbook causal linear attention:
    S_T = sum_s b_s k_s v_s^T, o = tril(Q K^T Diag(b)) V."""
    T, H, dk, dv = 11, 1, 16, 5
    rng = _rng(14)
    # rows of a 16x16 Sylvester-Hadamard matrix / 4, random signs and order:
    # orthonormal with every entry exact in binary floating point
    Hm = np.array([[1.0]])
    while Hm.shape[0] < dk:
        Hm = np.block([[Hm, Hm], [Hm, -Hm]])
    Hm = Hm * rng.choice([-1.0, 1.0], size=dk)[None, :] / 4.0
    k = Hm[rng.permutation(dk)[:T]][:, None, :]
    q = _f32(rng.standard_normal((T, H, dk)))
    v = _f32(rng.standard_normal((T, H, dv)))
    g = np.zeros((T, H, dk))
    b = _f32(rng.uniform(0.1, 1.0, (T, H)))
    o, ht = run(q, k, v, g, b, None)
    K, Q, V, bb = k[:, 0], q[:, 0], v[:, 0], b[:, 0]
    o_ref = np.tril(Q @ K.T * bb[None, :]) @ V
    assert np.allclose(o[:, 0], o_ref, rtol=1e-12, atol=1e-13), "P5 o"
    S_ref = (K * bb[:, None]).T @ V
    assert np.allclose(ht[0, 0], S_ref, rtol=1e-12, atol=1e-13), "P5 ht"


def pin_p6_write_then_read(run):
    """P6: beta = 1, ||k|| = 1, q = k gives o_t = v_t for any state (the
    token just written is read back exactly).  Keys are +-1/8 in 64 dims, so
    ||k|| = 1 exactly in binary arithmetic."""
    T, H, dk, dv = 10, 2, 64, 7
    rng = _rng(15)
    k = rng.choice([-0.125, 0.125], size=(T, H, dk))
    q = k.copy()
    v = _f32(rng.standard_normal((T, H, dv)))
    g = _f32(rng.uniform(-5.0, 0.0, (T, H, dk)))
    b = np.ones((T, H))
    h0 = rng.standard_normal((1, H, dk, dv))
    o, _ = run(q, k, v, g, b, h0)
    assert np.allclose(o, v, rtol=1e-12, atol=1e-12), "P6"


def pin_p8_affine_segments(run):
    """P8: a segment is an affine map of its incoming state,
    S_out(h) = M_seg h + S_out(0): linear in h, and composing two segments
    equals the whole run, while the plain sum of zero-start segment states
    (linear attention's shortcut) is wrong (Kimi K3 blog post, serving-stack
    section on splitting a sequence across devices).  Slow decay, so that
    M_seg does not vanish."""
    T, H, dk, dv = 24, 1, 6, 4
    rng = _rng(16)
    q = _f32(_unit(rng, (T, H, dk)))
    k = _f32(_unit(rng, (T, H, dk)))
    v = _f32(rng.standard_normal((T, H, dv)))
    g = _f32(rng.uniform(-0.05, 0.0, (T, H, dk)))
    b = _f32(rng.uniform(0.0, 1.0, (T, H)))
    h1 = rng.standard_normal((1, H, dk, dv))
    h2 = rng.standard_normal((1, H, dk, dv))
    _, s0 = run(q, k, v, g, b, None)
    _, s1 = run(q, k, v, g, b, h1)
    _, s2 = run(q, k, v, g, b, h2)
    _, s12 = run(q, k, v, g, b, 2.0 * h1 - 3.0 * h2)
    assert np.allclose(s12 - s0, 2.0 * (s1 - s0) - 3.0 * (s2 - s0), rtol=1e-11, atol=1e-12), "P8 linear"
    # transition of the second half from basis states, then composition
    T1 = 10
    sl = slice(T1, T)
    _, a_zero = run(q[:T1], k[:T1], v[:T1], g[:T1], b[:T1], h1)
    _, b_zero = run(q[sl], k[sl], v[sl], g[sl], b[sl], None)
    M = np.zeros((dk, dk))
    for c in range(dk):
        e = np.zeros((1, H, dk, dv))
        e[0, 0, c, 0] = 1.0
        _, sc = run(q[sl], k[sl], v[sl], g[sl], b[sl], e)
        M[:, c] = (sc - b_zero)[0, 0, :, 0]
    composed = M @ a_zero[0, 0] + b_zero[0, 0]
    assert np.allclose(composed, s1[0, 0], rtol=1e-11, atol=1e-12), "P8 compose"
    _, a0 = run(q[:T1], k[:T1], v[:T1], g[:T1], b[:T1], None)
    naive = a0[0, 0] + b_zero[0, 0]
    assert rel_l2(naive, s0[0, 0]) > 1e-2, "P8: the plain sum must be wrong"


def pin_p9_neutral_padding(run):
    """P9: tokens with g = 0 and beta = 0 (any q, k, v) leave the state
    unchanged, so inserting them changes neither later outputs nor ht."""
    T, H, dk, dv = 11, 2, 5, 4
    q, k, v, g, b, h0 = rand_case(17, T, H, dk, dv)
    o, ht = run(q, k, v, g, b, h0)
    rng = _rng(18)
    P = 5
    pos = 6
    ins = lambda a, x: np.concatenate([a[:pos], x, a[pos:]])
    q2 = ins(q, rng.standard_normal((P, H, dk)))
    k2 = ins(k, rng.standard_normal((P, H, dk)))
    v2 = ins(v, rng.standard_normal((P, H, dv)))
    g2 = ins(g, np.zeros((P, H, dk)))
    b2 = ins(b, np.zeros((P, H)))
    o2, ht2 = run(q2, k2, v2, g2, b2, h0)
    assert np.allclose(ht2, ht, rtol=1e-13, atol=1e-14), "P9 ht"
    assert np.allclose(o2[:pos], o[:pos], rtol=1e-13, atol=1e-14), "P9 o before"
    assert np.allclose(o2[pos + P:], o[pos:], rtol=1e-13, atol=1e-14), "P9 o after"


def pin_p10_varlen(run):
    """P10: packed sequences (cu_seqlens) equal separate runs."""
    H, dk, dv = 2, 4, 3
    lens = [5, 0, 9, 1]
    T = sum(lens)
    q, k, v, g, b, _ = rand_case(19, T, H, dk, dv)
    h0 = _rng(20).standard_normal((len(lens), H, dk, dv))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, ht = run(q, k, v, g, b, h0, cu)
    for n in range(len(lens)):
        sl = slice(cu[n], cu[n + 1])
        on, hn = run(q[sl], k[sl], v[sl], g[sl], b[sl], h0[n:n + 1])
        assert np.allclose(o[sl], on, rtol=1e-13, atol=1e-14), "P10 o"
        assert np.allclose(ht[n], hn[0], rtol=1e-13, atol=1e-14), "P10 ht"


def pin_p12_resume(run):
    """P12: prefill(T) == prefill(T1) then prefill(T - T1, h0 = ht_1)."""
    T, H, dk, dv = 20, 2, 5, 6
    q, k, v, g, b, h0 = rand_case(21, T, H, dk, dv, g_lo=-0.3)
    o, ht = run(q, k, v, g, b, h0)
    T1 = 7
    oa, ha = run(q[:T1], k[:T1], v[:T1], g[:T1], b[:T1], h0)
    ob, hb = run(q[T1:], k[T1:], v[T1:], g[T1:], b[T1:], ha)
    assert np.allclose(np.concatenate([oa, ob]), o, rtol=1e-12, atol=1e-13), "P12 o"
    assert np.allclose(hb, ht, rtol=1e-12, atol=1e-13), "P12 ht"


def pin_p1_chunked(run):
    """P1: the chunk-wise WY/UT form with the 16-token tile reference
    factoring (and the split intra/state output) reaches the token loop's
    result, for chunks of 16 and 64, a ragged tail, and g at the -5 floor."""
    T, H, dk, dv = 83, 2, 8, 6
    for g_lo, seed in ((-5.0, 22), (-0.05, 23)):
        q, k, v, g, b, h0 = rand_case(seed, T, H, dk, dv, g_lo=g_lo)
        o, ht = run(q, k, v, g, b, h0)
        for chunk in (16, 64):
            for split in (False, True):
                oc, hc = chunked_prefill(q, k, v, g, b, h0, chunk=chunk, split_output=split)
                assert rel_l2(oc, o) < 1e-12, ("P1 o", chunk, split)
                assert rel_l2(hc, ht) < 1e-12, ("P1 ht", chunk, split)
    # every log-decay at the floor: exp(80) is reached on the diagonal tiles
    q, k, v, g, b, h0 = rand_case(24, 64, 1, 8, 4)
    g = np.full_like(g, -5.0)
    o, ht = run(q, k, v, g, b, h0)
    oc, hc = chunked_prefill(q, k, v, g, b, h0, chunk=64, split_output=True)
    assert np.all(np.isfinite(oc)) and rel_l2(oc, o) < 1e-11, "P1 floor"


PINS = [pin_p1_chunked, pin_p2_bruteforce, pin_p3_beta_zero, pin_p4_one_hot,
        pin_p5_orthonormal, pin_p6_write_then_read, pin_p8_affine_segments,
        pin_p9_neutral_padding, pin_p10_varlen, pin_p12_resume]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
@pytest.mark.parametrize("runner", [run_c, run_np], ids=["c", "numpy"])
def test_pin(pin, runner):
    pin(runner)


# ------------------------------------------------- oracle-only ablation (P7)

def test_p7_gla_ablation():
    """P7: with the erase term switched off the recurrence is gated linear
    attention: o_t = sum_{s<=t} ((q_t * e^{Gam_t - Gam_s}) . k_s) b_s v_s;
    at g = 0, b = 1 this is the causal prefix sum o = tril(Q K^T) V."""
    T, H, dk, dv = 9, 2, 5, 4
    q, k, v, g, b, _ = rand_case(25, T, H, dk, dv, g_lo=-1.0)
    o, _ = oracle.prefill(q, k, v, g, b, None, None, flags=oracle.NO_ERASE)
    o2, _ = oracle.prefill_np(q, k, v, g, b, None, None, erase=False)
    Gam = np.cumsum(g, axis=0)
    for h in range(H):
        for t in range(T):
            ref = sum(np.dot(q[t, h] * np.exp(Gam[t, h] - Gam[s, h]), k[s, h]) * b[s, h] * v[s, h]
                      for s in range(t + 1))
            assert np.allclose(o[t, h], ref, rtol=1e-12, atol=1e-13)
            assert np.allclose(o2[t, h], ref, rtol=1e-12, atol=1e-13)
    o, _ = oracle.prefill(q, k, v, np.zeros_like(g), np.ones_like(b), None, None,
                          flags=oracle.NO_ERASE)
    for h in range(H):
        ref = np.tril(q[:, h] @ k[:, h].T) @ v[:, h]
        assert np.allclose(o[:, h], ref, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------ decode (P13) and C/np

def test_p13_prefill_equals_decode_steps():
    """P13: a prefill over T tokens equals T decode steps on the same state."""
    T, H, dk, dv = 13, 3, 6, 5
    q, k, v, g, b, h0 = rand_case(26, T, H, dk, dv)
    o, ht = oracle.prefill(q, k, v, g, b, h0)
    state = np.array(h0, dtype=np.float64)   # N = 1
    state2 = state.copy()
    for t in range(T):
        ot = oracle.decode_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], b[t:t + 1], state)
        ot2 = oracle.decode_step_np(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], b[t:t + 1], state2)
        assert np.allclose(ot[0], o[t], rtol=1e-12, atol=1e-13)
        assert np.allclose(ot2[0], o[t], rtol=1e-12, atol=1e-13)
    assert np.allclose(state, ht, rtol=1e-12, atol=1e-13)
    assert np.allclose(state2, ht, rtol=1e-12, atol=1e-13)


def test_c_matches_numpy_twin():
    """The C loop and the numpy twin agree on a mixed varlen case."""
    H, dk, dv = 3, 16, 12
    lens = [17, 1, 40, 0, 33]
    T = sum(lens)
    q, k, v, g, b, _ = rand_case(27, T, H, dk, dv)
    h0 = _rng(28).standard_normal((len(lens), H, dk, dv))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o1, s1 = oracle.prefill(q, k, v, g, b, h0, cu)
    o2, s2 = oracle.prefill_np(q, k, v, g, b, h0, cu)
    assert rel_l2(o1, o2) < 1e-13 and rel_l2(s1, s2) < 1e-13


def test_hand_worked_scalar():
    """dk = dv = 1 worked by hand.  h0 = 4.
    t=1: k=1, b=1/2, v=2, e^g=1/2, q=1:  S = (1-1/2)(1/2)4 + (1/2)(1)(2) = 2, o = 2.
    t=2: k=1/2, b=1, v=-4, g=0, q=2:   S = (1-1/4)2 + (1)(1/2)(-4) = -1/2, o = -1."""
    q = np.array([[[1.0]], [[2.0]]])
    k = np.array([[[1.0]], [[0.5]]])
    v = np.array([[[2.0]], [[-4.0]]])
    g = np.array([[[math.log(0.5)]], [[0.0]]])
    b = np.array([[0.5], [1.0]])
    h0 = np.array([[[[4.0]]]])
    o, ht = oracle.prefill(q, k, v, g, b, h0)
    # float32 rounding of ln(1/2) perturbs e^g by < 1e-7
    assert abs(o[0, 0, 0] - 2.0) < 1e-6 and abs(o[1, 0, 0] + 1.0) < 1e-6
    assert abs(ht[0, 0, 0, 0] + 0.5) < 1e-6


# -------------------------------------------------------- decay bound (P11)

def test_p11_decay_bound_numbers():
    """The numbers of the blog post's decay-bound section (golden fixture):
    keeping at least 0.67% per step means g >= -5 (natural log); a 16-token
    tile then sums to at least -80; e^80 ~ 5.5e34 is below bf16's ~3.4e38."""
    with open(os.path.join(GOLDEN, "decay_bound.json")) as f:
        gold = json.load(f)
    floor = gold["per_step_log_decay_floor"]
    assert round(100 * math.exp(floor), 2) == gold["per_step_retention_floor_percent"]
    assert math.log(gold["per_step_retention_floor_percent"] / 100) == pytest.approx(floor, abs=0.01)
    lo = gold["tile_tokens"] * floor
    assert lo == gold["tile_cumulative_log_decay_interval"][0]
    assert math.exp(-lo) == pytest.approx(gold["reciprocal_bound"], rel=0.01)
    bf16_max = float(torch.finfo(torch.bfloat16).max)
    assert bf16_max == pytest.approx(gold["bf16_range"], rel=0.01)
    assert math.exp(-lo) < bf16_max
    # and the bf16 cast of e^80 is finite
    assert torch.isfinite(torch.tensor(math.exp(80.0)).to(torch.bfloat16)).item()


@pytest.mark.parametrize("mode", workloads.G_MODES)
def test_p11_generated_tiles_respect_bound(mode):
    """Every 16-token tile aligned to a chunk / sequence start of every
    generated input has per-channel sum of g in [-80, 0]."""
    spec = workloads.PrefillSpec(H=3, dk=16, dv=8, seqlens=(37, 64, 5, 130),
                                 g_mode=mode, seed=5)
    x = workloads.make_prefill(spec)
    g = x["g"][0].numpy().astype(np.float64)
    assert g.min() >= -5.0 and g.max() <= 0.0
    cu = x["cu_seqlens"].numpy()
    for n in range(len(cu) - 1):
        for t0 in range(cu[n], cu[n + 1], 16):
            s = g[t0:min(t0 + 16, cu[n + 1])].sum(axis=0)
            assert s.min() >= -80.0 and s.max() <= 0.0


# ---------------------------------------------- the pins catch planted bugs

def _mutant(kind):
    """numpy token loops, each with one planted mistake."""
    def run(q, k, v, g, beta, h0=None, cu=None):
        q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
        T, H, dk = q.shape
        dv = v.shape[-1]
        cu = [0, T] if cu is None else [int(c) for c in cu]
        o = np.zeros((T, H, dv))
        ht = np.zeros((len(cu) - 1, H, dk, dv))
        for n in range(len(cu) - 1):
            S = np.zeros((H, dk, dv)) if h0 is None else np.array(h0[n], dtype=np.float64)
            for t in range(cu[n], cu[n + 1]):
                kt, qt, vt, gt, bt = k[t], q[t], v[t], g[t], beta[t][:, None, None]
                dec = np.exp(gt)[:, :, None]
                if kind == "read_before_update":
                    o[t] = np.einsum("hcj,hc->hj", dec * S, qt)
                if kind == "decay_after_erase":
                    kS = np.einsum("hc,hcj->hj", kt, S)
                    S = S - bt * kt[:, :, None] * kS[:, None, :]
                    S = dec * S
                else:
                    S = dec * S if kind != "decay_columns" else S * np.exp(gt[:, :dv])[:, None, :]
                    kS = np.einsum("hc,hcj->hj", kt, S)
                    sign = -1.0 if kind != "erase_sign" else 1.0
                    erase_b = bt if kind != "erase_no_beta" else 1.0
                    S = S + sign * erase_b * kt[:, :, None] * kS[:, None, :]
                wb = bt if kind != "write_no_beta" else 1.0
                S = S + wb * kt[:, :, None] * vt[:, None, :]
                if kind == "read_with_k":
                    o[t] = np.einsum("hcj,hc->hj", S, kt)
                elif kind != "read_before_update":
                    o[t] = np.einsum("hcj,hc->hj", S, qt)
            ht[n] = S
        return o, ht
    return run


MUTANTS = ["read_before_update", "decay_after_erase", "decay_columns",
           "erase_sign", "erase_no_beta", "write_no_beta", "read_with_k"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_catch_planted_mistakes(kind):
    run = _mutant(kind)
    failed = []
    for pin in PINS:
        try:
            pin(run)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {kind!r}"
